// Budgeted community retrieval (the CommunityKV page, Figure 1 panel (3):
// retrieve a candidate subset of communities under a token budget).
//
// One 1024-thread block per graph.  Every community becomes a 64-bit key,
// (order-preserving bits of its float32 score) << 32 | (~id), so a larger key
// means a better rank and ties of the score fall to the lower id.  The taken
// set is the longest prefix of the ranking that fits the budget, i.e. every key
// above the key of the first community that overflows it.
//
// The cut is found in two steps.  First a token-weighted histogram over 1024
// equal-width score bins between the lowest and highest score (a monotone map
// of the score, so bins keep the ranking) and one block scan from the top bin
// give the bin holding the cut; every community above it is taken.  Then the
// few communities of that bin are sorted by key in one wave (bitonic network)
// and walked until the budget overflows.  When the scores are degenerate (all
// equal, or more than 64 in the cut bin) a most-significant-digit radix select
// over the keys with token-weighted digit histograms finds the same cut.  The
// community cap (max_comm) is the same radix select with unit weights.
//
// Then the taken ids are compacted in ascending id order with block scans, and
// the attended token list is written: sinks, the base members of every taken
// community, then the taken communities' tail members.  Sizes, scores and tail
// entries are read at the start with 16-byte loads; CSR offsets only for the
// taken communities.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kBins = kSelThreads;
// Taken communities whose copy runs block-wide out of LDS (more fall back to
// one thread per community).
constexpr int kSelLds = 4096;
constexpr int kTailPerThread = 4;  // tail_cap <= 4096

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

struct SelShared {
    int sid[kSelLds];        // taken community
    int soff[kSelLds];       // its first base member in toks
    int spref[kSelLds + 1];  // its first slot in the token list (after the sinks)
    int bw[kBins];           // token weight per score bin
    uint32_t hw[256];        // radix fallback: token weight per digit
    uint32_t hn[256];        // radix fallback: candidates per digit
    uint32_t bits[CKV_MAX_C_CAP / 32];
    unsigned long long ckey[64];
    int csz[64];
    int ccount;
    int cut_bin, cut_above;
    int scan[kSelThreads / 64 + 1];
    unsigned long long red_max[kSelThreads / 64];
    unsigned long long red_min[kSelThreads / 64];
    unsigned long long prefix, mask, thr;
    long long rem;
    int done;
};

__device__ __forceinline__ float key_score(unsigned long long k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Threshold key of the budget cut by radix select over the keys: the taken
// communities are those with key > threshold (0 = everything fits).  `unit`
// counts communities instead of tokens (the community cap).
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

// Budget cut through equal-width score bins (see the file comment).  Returns
// false, uniformly across the block, when the radix select has to decide.
template <int EPT>
__device__ bool value_cut(const unsigned long long (&key)[EPT], const float (&sv)[EPT], const int (&w)[EPT],
                          int budget, unsigned long long kmax, unsigned long long kmin, SelShared &sh,
                          unsigned long long &thr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float hi = key_score(kmax), lo = key_score(kmin);
    const float scale = (float)kBins / (hi - lo);
    if (!(hi > lo) || !(scale < __builtin_huge_valf())) return false;
    sh.bw[tid] = 0;
    if (tid == 0) {
        sh.ccount = 0;
        sh.cut_bin = -1;
    }
    __syncthreads();
    int bin[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        bin[j] = -1;
        if (key[j]) {
            bin[j] = min(kBins - 1, (int)((sv[j] - lo) * scale));
            atomicAdd(&sh.bw[bin[j]], w[j]);
        }
    }
    __syncthreads();
    const int rb = kBins - 1 - tid;  // thread t scans bins from the top
    const int v = sh.bw[rb];
    int total;
    const int excl = block_exclusive_scan<kSelThreads>(v, sh.scan, &total);
    if (total <= budget) {  // every community fits
        thr = 0ull;
        __syncthreads();
        return true;
    }
    if (excl <= budget && budget < excl + v) {
        sh.cut_bin = rb;
        sh.cut_above = excl;
    }
    __syncthreads();
    const int cb = sh.cut_bin, above = sh.cut_above;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (bin[j] == cb) {
            const int i = atomicAdd(&sh.ccount, 1);
            if (i < 64) {
                sh.ckey[i] = key[j];
                sh.csz[i] = w[j];
            }
        }
    }
    __syncthreads();
    const int cnt = sh.ccount;
    if (cnt > 64) {
        __syncthreads();
        return false;
    }
    if (wave == 0) {
        // bitonic sort of the complemented keys, ascending = keys descending
        unsigned long long nk = lane < cnt ? ~sh.ckey[lane] : ~0ull;
        int sz = lane < cnt ? sh.csz[lane] : 0;
#pragma unroll
        for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
            for (int jj = k >> 1; jj > 0; jj >>= 1) {
                const unsigned long long onk = __shfl_xor(nk, jj, 64);
                const int osz = __shfl_xor(sz, jj, 64);
                const bool lower = (lane & jj) == 0;
                const bool asc = (lane & k) == 0;
                const bool take = (lower == asc) ? (onk < nk) : (onk > nk);
                if (take) {
                    nk = onk;
                    sz = osz;
                }
            }
        }
        int incl = sz;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const unsigned long long bal = __ballot(lane < cnt && above + incl > budget);
        const int first = bal ? __ffsll((long long)bal) - 1 : 0;
        const unsigned long long cut = ~__shfl(nk, first, 64);
        if (lane == 0) sh.thr = cut;
    }
    __syncthreads();
    thr = sh.thr;
    __syncthreads();
    return true;
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

    // Sizes and scores of this thread's EPT consecutive communities, 16 bytes
    // per load; the tail entries too.  (CSR offsets are fetched later, for the
    // taken communities only.)
    static_assert(EPT % 4 == 0, "EPT must be a multiple of 4");
    int s[EPT];
    float sv[EPT];
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
        const int c = tid * EPT + j;  // c % 4 == 0 and C % 256 == 0: the load stays in the row
        int4 s4 = make_int4(0, 0, 0, 0);
        float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < nc) {
            s4 = *reinterpret_cast<const int4 *>(sz + c);
            v4 = *reinterpret_cast<const float4 *>(sc + c);
        }
        s[j] = c < nc ? s4.x : 0;
        s[j + 1] = c + 1 < nc ? s4.y : 0;
        s[j + 2] = c + 2 < nc ? s4.z : 0;
        s[j + 3] = c + 3 < nc ? s4.w : 0;
        sv[j] = v4.x;
        sv[j + 1] = v4.y;
        sv[j + 2] = v4.z;
        sv[j + 3] = v4.w;
    }
    const int tn = p.tail_len[g];
    int tcomm[kTailPerThread], tpos[kTailPerThread];
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
        const int i = tid * kTailPerThread + j;
        const bool in = i < p.tail_cap;
        tcomm[j] = in ? p.tail_comm[(size_t)g * p.tail_cap + i] : -1;
        tpos[j] = in ? p.tail_pos[(size_t)g * p.tail_cap + i] : 0;
    }

    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;

    unsigned long long key[EPT];
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid * EPT + j;
        if (sv[j] == 0.f) sv[j] = 0.f;  // one key for +0 and -0
        key[j] = (s[j] > 0) ? (((unsigned long long)ordered_bits(sv[j]) << 32) | (0xFFFFFFFFu - (uint32_t)c)) : 0ull;
        if (key[j]) {
            kmax = umax64(kmax, key[j]);
            kmin = umin64(kmin, key[j]);
        }
    }
    kmax = wave_max_u64(kmax);
    kmin = wave_min_u64(kmin);
    if (lane == 0) {
        sh.red_max[wave] = kmax;
        sh.red_min[wave] = kmin;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        kmax = umax64(kmax, sh.red_max[i]);
        kmin = umin64(kmin, sh.red_min[i]);
    }
    __syncthreads();

    unsigned long long thr = ~0ull;  // nothing taken when there is no candidate
    if (kmax != 0ull) {
        if (!value_cut<EPT>(key, sv, s, p.budget, kmax, kmin, sh, thr))
            thr = radix_cut<EPT>(key, s, false, (long long)p.budget, kmax, kmin, sh);
        if (p.max_comm > 0) {
            const unsigned long long t2 = radix_cut<EPT>(key, s, true, (long long)p.max_comm, kmax, kmin, sh);
            thr = t2 > thr ? t2 : thr;
        }
    }

    // Compact the taken ids (ascending) and give each its slot in tok_list.
    int nloc = 0, tokloc = 0;
    int o0[EPT], o1[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid * EPT + j;
        const bool t = key[j] > thr;
        o0[j] = t ? offs[c] : 0;
        o1[j] = t ? offs[c + 1] : 0;
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (key[j] > thr) {
            ++nloc;
            tokloc += o1[j] - o0[j];
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
            if (staged) {
                sh.sid[kpos] = c;
                sh.soff[kpos] = o0[j];
                sh.spref[kpos] = dst - ns;
            } else {
                for (int i = o0[j]; i < o1[j]; ++i) tl[dst + i - o0[j]] = toks[i];
            }
            dst += o1[j] - o0[j];
            ++kpos;
        }
    }
    if (tid == 0 && staged) sh.spref[nsel] = ntok;
    for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
    __syncthreads();
    if (staged) {
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

    // Tail members of taken communities, in tail order.
    int f[kTailPerThread], floc = 0;
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
        const int i = tid * kTailPerThread + j;
        const int c = tcomm[j];
        f[j] = (i < tn && c >= 0 && c < C && ((sh.bits[c >> 5] >> (c & 31)) & 1u)) ? 1 : 0;
        floc += f[j];
    }
    int ntail;
    int tdst = ns + ntok + block_exclusive_scan<kSelThreads>(floc, sh.scan, &ntail);
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j)
        if (f[j]) tl[tdst++] = tpos[j];

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
    if (ept <= 4) hipLaunchKernelGGL((select_kernel<4>), grid, block, 0, s, p);
    else if (ept <= 8) hipLaunchKernelGGL((select_kernel<8>), grid, block, 0, s, p);
    else if (ept <= 12) hipLaunchKernelGGL((select_kernel<12>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((select_kernel<16>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace ckv
