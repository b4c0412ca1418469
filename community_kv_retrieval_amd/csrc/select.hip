// Budgeted community retrieval (the CommunityKV page, Figure 1 panel (3):
// retrieve a candidate subset of communities under a token budget).
//
// One 1024-thread block per graph.  Every community becomes a 64-bit key,
// (order-preserving bits of its float32 score) << 32 | (~id), so a larger key
// means a better rank and ties of the score fall to the lower id.  The taken
// set is the longest prefix of the ranking that fits the budget, i.e. every key
// above the key of the first community that overflows it.  That cut is found
// with a most-significant-digit radix select over the keys whose histogram
// counts member tokens instead of keys: starting at the highest bit where the
// candidates differ, each 8-bit pass builds the token-weighted histogram of
// the remaining candidates in LDS, one wave walks it from the top to find the
// digit where the running total passes the remaining budget, and the
// candidates narrow to that digit.  It stops as soon as one candidate is left.
// The community cap (max_comm) is the same select with unit weights.
// The taken ids are then compacted in ascending id order with a block scan,
// and the attended token list is written: sinks, the base members of every
// taken community, then the taken communities' tail members.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;

struct SelectParams {
    const float *scores;
    const int32_t *size;
    const int32_t *offs;
    const int32_t *toks;
    const int32_t *tail_pos;
    const int32_t *tail_comm;
    const int32_t *tail_len;
    const int32_t *n_comm;
    const int32_t *seq_len;
    int mode, Hq, Hkv, c_cap, l_cap, tail_cap, n_sinks, budget, max_comm, t_cap;
    int32_t *sel;
    int32_t *sel_n;
    int32_t *top;
    int32_t *tok_list;
    int32_t *tok_n;
};

// Taken communities whose copy runs block-wide out of LDS (more fall back to
// one thread per community).
constexpr int kSelLds = 4096;

struct SelShared {
    int sid[kSelLds];      // taken community
    int soff[kSelLds];     // its first base member in toks
    int spref[kSelLds + 1];  // its first slot in the token list (after the sinks)
    uint32_t hw[256];  // token weight per digit
    uint32_t hn[256];  // candidates per digit
    uint32_t bits[CKV_MAX_C_CAP / 32];
    int scan[kSelThreads / 64 + 1];
    unsigned long long red_max[kSelThreads / 64];
    unsigned long long red_min[kSelThreads / 64];
    unsigned long long prefix, mask;
    long long rem;
    int done;
};

__device__ __forceinline__ uint32_t ordered_bits(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Threshold key of the budget cut: the taken communities are those with
// key > threshold (0 = everything fits).  `unit` counts communities instead of
// tokens (the community cap).
template <int EPT>
__device__ unsigned long long radix_cut(const unsigned long long (&key)[EPT], const int (&w)[EPT],
                                        bool unit, long long budget, unsigned long long kmax,
                                        unsigned long long kmin, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned long long diff = kmax ^ kmin;
    int hi = diff ? 63 - __clzll((long long)diff) : 0;
    unsigned long long mask = ~((2ull << hi) - 1ull);  // bits above hi (0 when hi == 63)
    unsigned long long prefix = kmax & mask;
    long long rem = budget;
    for (;;) {
        const int lo = hi >= 7 ? hi - 7 : 0;
        const uint32_t dm = (1u << (hi - lo + 1)) - 1u;
        if (tid < 256) {
            sh.hw[tid] = 0;
            sh.hn[tid] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (key[j] && (key[j] & mask) == prefix) {
                const uint32_t d = (uint32_t)(key[j] >> lo) & dm;
                atomicAdd(&sh.hw[d], unit ? 1u : (uint32_t)w[j]);
                atomicAdd(&sh.hn[d], 1u);
            }
        }
        __syncthreads();
        if (wave == 0) {
            long long h[4], tot = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = sh.hw[4 * lane + i];
                tot += h[i];
            }
            long long suf = tot;  // sum over this lane and every higher lane
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const long long y = __shfl_down(suf, o, 64);
                if (lane + o < 64) suf += y;
            }
            long long accw = suf - tot, above = 0;
            int found = -1;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                if (found < 0 && accw + h[i] > rem) {
                    found = 4 * lane + i;
                    above = accw;
                }
                accw += h[i];
            }
            const unsigned long long bal = __ballot(found >= 0);
            const int src = bal ? 63 - __clzll((long long)bal) : 0;
            const int d = __shfl(found, src, 64);
            const long long ab = __shfl(above, src, 64);
            if (lane == 0) {
                if (bal == 0) {
                    sh.done = 2;
                } else {
                    sh.rem = rem - ab;
                    sh.prefix = prefix | ((unsigned long long)d << lo);
                    sh.mask = mask | ((unsigned long long)dm << lo);
                    sh.done = (sh.hn[d] == 1u || lo == 0) ? 1 : 0;
                }
            }
        }
        __syncthreads();
        const int done = sh.done;
        if (done == 2) {
            __syncthreads();
            return 0ull;
        }
        prefix = sh.prefix;
        mask = sh.mask;
        rem = sh.rem;
        __syncthreads();
        if (done == 1) return prefix | ~mask;
        hi = lo - 1;
    }
}

template <int EPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
    __shared__ SelShared sh;
    const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = p.c_cap;
    const int nc = min(p.n_comm[g], C);
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int L = p.seq_len[gc.b];
    const int ns = min(p.n_sinks, max(L, 0));
    const float *sc = p.scores + (size_t)g * C;
    const int32_t *sz = p.size + (size_t)g * C;
    const int32_t *offs = p.offs + (size_t)g * (C + 1);
    int32_t *tl = p.tok_list + (size_t)g * p.t_cap;

    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;

    unsigned long long key[EPT];
    int w[EPT];
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid * EPT + j;
        const int s = (c < nc) ? sz[c] : 0;
        float v = (s > 0) ? sc[c] : 0.f;
        if (v == 0.f) v = 0.f;  // one key for +0 and -0
        key[j] = (s > 0) ? (((unsigned long long)ordered_bits(v) << 32) | (0xFFFFFFFFu - (uint32_t)c)) : 0ull;
        w[j] = s;
        if (key[j]) {
            kmax = key[j] > kmax ? key[j] : kmax;
            kmin = key[j] < kmin ? key[j] : kmin;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long a = __shfl_xor(kmax, o, 64), b = __shfl_xor(kmin, o, 64);
        kmax = a > kmax ? a : kmax;
        kmin = b < kmin ? b : kmin;
    }
    if (lane == 0) {
        sh.red_max[wave] = kmax;
        sh.red_min[wave] = kmin;
    }
    __syncthreads();
    kmax = 0ull;
    kmin = ~0ull;
    for (int i = 0; i < kSelThreads / 64; ++i) {
        kmax = sh.red_max[i] > kmax ? sh.red_max[i] : kmax;
        kmin = sh.red_min[i] < kmin ? sh.red_min[i] : kmin;
    }
    __syncthreads();

    unsigned long long thr = ~0ull;  // nothing taken when there is no candidate
    if (kmax != 0ull) {
        thr = radix_cut<EPT>(key, w, false, (long long)p.budget, kmax, kmin, sh);
        if (p.max_comm > 0) {
            const unsigned long long t2 = radix_cut<EPT>(key, w, true, (long long)p.max_comm, kmax, kmin, sh);
            thr = t2 > thr ? t2 : thr;
        }
    }

    // Compact the taken ids (ascending) and give each its slot in tok_list.
    int nloc = 0, tokloc = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (key[j] > thr) {
            const int c = tid * EPT + j;
            ++nloc;
            tokloc += offs[c + 1] - offs[c];
        }
    }
    int nsel, ntok;
    int kpos = block_exclusive_scan<kSelThreads>(nloc, sh.scan, &nsel);
    __syncthreads();
    int dst = ns + block_exclusive_scan<kSelThreads>(tokloc, sh.scan, &ntok);
    __syncthreads();
    const int32_t *toks = p.toks + (size_t)g * p.l_cap;
    const bool staged = nsel <= kSelLds;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (key[j] > thr) {
            const int c = tid * EPT + j;
            p.sel[(size_t)g * C + kpos] = c;
            atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
            const int o = offs[c], e = offs[c + 1];
            if (staged) {
                sh.sid[kpos] = c;
                sh.soff[kpos] = o;
                sh.spref[kpos] = dst - ns;
            } else {
                for (int i = o; i < e; ++i) tl[dst + i - o] = toks[i];
            }
            dst += e - o;
            ++kpos;
        }
    }
    if (staged) {
        if (tid == 0) sh.spref[nsel] = ntok;
        __syncthreads();
        // slot j of the member part belongs to the last taken community whose
        // first slot is <= j
        for (int j0 = 0; j0 < ntok; j0 += 4 * kSelThreads) {
            int v[4], at[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                at[u] = j;
                if (j < ntok) {
                    int lo = 0, hi = nsel - 1;
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (sh.spref[mid] <= j) lo = mid;
                        else hi = mid - 1;
                    }
                    v[u] = toks[sh.soff[lo] + (j - sh.spref[lo])];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (at[u] < ntok) tl[ns + at[u]] = v[u];
        }
    }
    for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
    __syncthreads();

    // Tail members of taken communities, in tail order.
    const int tn = p.tail_len[g];
    constexpr int TPT = 4;  // tail_cap <= 4096
    int f[TPT], floc = 0;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        const int i = tid * TPT + j;
        f[j] = 0;
        if (i < tn) {
            const int c = p.tail_comm[(size_t)g * p.tail_cap + i];
            f[j] = (c >= 0 && c < C && ((sh.bits[c >> 5] >> (c & 31)) & 1u)) ? 1 : 0;
        }
        floc += f[j];
    }
    int ntail;
    int tdst = ns + ntok + block_exclusive_scan<kSelThreads>(floc, sh.scan, &ntail);
#pragma unroll
    for (int j = 0; j < TPT; ++j)
        if (f[j]) tl[tdst++] = p.tail_pos[(size_t)g * p.tail_cap + tid * TPT + j];

    if (tid == 0) {
        p.sel_n[g] = nsel;
        p.tok_n[g] = ns + ntok + ntail;
        p.top[g] = kmax ? (int)(0xFFFFFFFFu - (uint32_t)kmax) : -1;
    }
}

hipError_t launch_select(const ckv_kv *kv, const ckv_index *idx, const float *scores, int budget,
                         int max_comm, int t_cap, int32_t *sel, int32_t *sel_n, int32_t *top,
                         int32_t *tok_list, int32_t *tok_n, hipStream_t s) {
    SelectParams p{};
    p.scores = scores;
    p.size = idx->size;
    p.offs = idx->offs;
    p.toks = idx->toks;
    p.tail_pos = idx->tail_pos;
    p.tail_comm = idx->tail_comm;
    p.tail_len = idx->tail_len;
    p.n_comm = idx->n_comm;
    p.seq_len = kv->seq_len;
    p.mode = idx->mode;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.c_cap = idx->c_cap;
    p.l_cap = idx->l_cap;
    p.tail_cap = idx->tail_cap;
    p.n_sinks = idx->n_sinks;
    p.budget = budget;
    p.max_comm = max_comm;
    p.t_cap = t_cap;
    p.sel = sel;
    p.sel_n = sel_n;
    p.top = top;
    p.tok_list = tok_list;
    p.tok_n = tok_n;
    const int ept = ceil_div(idx->c_cap, kSelThreads);
    const dim3 grid(idx->n_graphs), block(kSelThreads);
    if (ept <= 1) hipLaunchKernelGGL((select_kernel<1>), grid, block, 0, s, p);
    else if (ept <= 2) hipLaunchKernelGGL((select_kernel<2>), grid, block, 0, s, p);
    else if (ept <= 4) hipLaunchKernelGGL((select_kernel<4>), grid, block, 0, s, p);
    else if (ept <= 8) hipLaunchKernelGGL((select_kernel<8>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((select_kernel<16>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace ckv
