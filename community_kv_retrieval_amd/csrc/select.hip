// Budgeted community retrieval (the CommunityKV page, Figure 1 panel (3):
// retrieve a candidate subset of communities under a token budget).
//
// One 1024-thread block per graph.  The communities are read in slabs of 4096:
// in slab j thread t owns communities 4096 j + 4 t .. 4096 j + 4 t + 3, so
// every 16-byte load of a wave covers 1 KB of consecutive memory.
// Communities rank by float32 score, higher first, ties to the lower id; as
// one number that is the 64-bit key (order-preserving bits of the score) << 32
// | (~id).  The taken set is the longest prefix of the ranking that fits the
// budget, i.e. every key above the key of the first community that overflows
// it (the cut).
//
// The whole graph runs on one CU, so the passes over every community use
// 32-bit arithmetic only.  The cut is found in two steps: a token-weighted
// histogram over 1024 equal-width score bins between the lowest and highest
// score (a monotone map of the score, so bins keep the ranking), walked from
// the top by one wave, gives the bin holding the cut; every community above it
// is taken.  The few communities of that bin get their 64-bit keys, one wave
// sorts them (bitonic network) and walks them until the budget overflows.
// When the scores are degenerate (all equal, or more than 64 in the cut bin) a
// most-significant-digit radix select over the 64-bit keys, with
// token-weighted digit histograms, finds the same cut.  The community cap
// (max_comm) is the same radix select with unit weights.
//
// Then one block scan over per-slab counts gives every taken community its
// rank in ascending id order and its first slot in the token list, and every
// taken tail entry its slot after them.  The list is written as sinks, the base
// members of every taken community (each slot finds its community by binary
// search over the communities' first slots), then the taken tail members in
// tail order.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kBins = kSelThreads;
constexpr int kSlab = 4 * kSelThreads;  // communities per slab
// Taken communities whose first slots are kept in LDS for the binary-search
// copy; more than that are copied one thread per community.
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
    int mode, Hq, Hkv, c_cap, l_cap, tail_cap, n_sinks, budget, max_comm, t_cap, g0;
    int32_t *sel;
    int32_t *sel_n;
    int32_t *top;
    int32_t *tok_list;
    int32_t *tok_n;
};

struct SelShared {
    int soff[kSelLds];       // first base member in toks of the k-th taken community
    int spref[kSelLds];      // its first slot in the token list (after the sinks)
    int bw[kBins];           // token weight per score bin
    uint32_t hw[256];        // radix select: token weight per digit
    uint32_t hn[256];        // radix select: candidates per digit
    uint32_t bits[CKV_MAX_C_CAP / 32];
    unsigned long long ckey[64];
    int csz[64];
    int ccount;
    int cut_bin, cut_above;
    int scan[(kSelThreads / 64) * 9];
    float red_lo[kSelThreads / 64], red_hi[kSelThreads / 64];
    uint32_t red_id[kSelThreads / 64];
    unsigned long long prefix, mask, thr;
    long long rem;
    int done;
};

__device__ __forceinline__ unsigned long long comm_key(float s, int c) {
    return ((unsigned long long)ordered_bits(s) << 32) | (0xFFFFFFFFu - (uint32_t)c);
}

// Community id of element e (0 .. 4 NS - 1) of thread tid.
__device__ __forceinline__ int slab_id(int tid, int e) { return (e >> 2) * kSlab + 4 * tid + (e & 3); }

// Block-wide exclusive prefix sums of NV ints per thread, in thread order, and
// their totals.  One barrier: every wave scans the wave totals itself.
// `scratch` holds NT/64 * NV ints; the caller puts a barrier between two uses.
template <int NT, int NV>
__device__ __forceinline__ void block_scan_multi(const int (&v)[NV], int (&ex)[NV], int (&tot)[NV], int *scratch) {
    constexpr int NW = NT / 64;
    static_assert(NW <= 64, "one lane per wave total");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k] = wave_incl_scan(v[k]);
    if (lane == 63) {
#pragma unroll
        for (int k = 0; k < NV; ++k) scratch[wave * NV + k] = x[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int t = lane < NW ? scratch[lane * NV + k] : 0;
        const int ti = wave_incl_scan(t);
        tot[k] = __builtin_amdgcn_readlane(ti, NW - 1);
        const int before = wave > 0 ? __builtin_amdgcn_readlane(ti, wave > 0 ? wave - 1 : 0) : 0;
        ex[k] = before + x[k] - v[k];
    }
}

// Threshold key of the budget cut by radix select over the 64-bit keys: the
// taken communities are those with key > threshold (0 = everything fits).
// `unit` counts communities instead of tokens (the community cap).
template <int EPT>
__device__ unsigned long long radix_cut(const float (&sv)[EPT], const int (&w)[EPT], bool unit,
                                        long long budget, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long key[EPT];
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        key[j] = w[j] > 0 ? comm_key(sv[j], slab_id(tid, j)) : 0ull;
        if (key[j]) {
            kmax = umax64(kmax, key[j]);
            kmin = umin64(kmin, key[j]);
        }
    }
    kmax = wave_max_u64(kmax);
    kmin = wave_min_u64(kmin);
    if (lane == 0) {
        sh.ckey[wave] = kmax;
        sh.ckey[32 + wave] = kmin;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        kmax = umax64(kmax, sh.ckey[i]);
        kmin = umin64(kmin, sh.ckey[32 + i]);
    }
    __syncthreads();
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

// Budget cut through equal-width score bins (see the file comment).  The bin
// weights and the candidate count must be zero on entry.  Returns false,
// uniformly across the block, when the radix select has to decide.
template <int EPT>
__device__ bool value_cut(const float (&sv)[EPT], const int (&w)[EPT], int budget, float lo, float hi,
                          SelShared &sh, unsigned long long &thr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float scale = (float)kBins / (hi - lo);
    if (!(hi > lo) || !(scale < __builtin_huge_valf())) return false;
    int bin[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        bin[j] = -1;
        if (w[j] > 0) {
            bin[j] = min(kBins - 1, (int)((sv[j] - lo) * scale));
            atomicAdd(&sh.bw[bin[j]], w[j]);
        }
    }
    __syncthreads();
    CKV_TMARK(40);
    // One wave walks the bins from the top: lane l owns bins
    // kBins-1-16l .. kBins-16-16l, a prefix over lanes gives each lane the
    // weight above its bins.
    if (wave == 0) {
        int v[16], tot = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            v[k] = sh.bw[kBins - 1 - (lane * 16 + k)];
            tot += v[k];
        }
        const int incl = wave_incl_scan(tot);
        int acc = incl - tot, found = -1, above = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (found < 0 && acc + v[k] > budget) {
                found = kBins - 1 - (lane * 16 + k);
                above = acc;
            }
            acc += v[k];
        }
        const unsigned long long bal = __ballot(found >= 0);
        const int src = bal ? __ffsll((long long)bal) - 1 : 0;
        const int fb = __shfl(found, src, 64), fa = __shfl(above, src, 64);
        if (lane == 0) {
            sh.cut_bin = bal ? fb : -1;  // -1: every community fits
            sh.cut_above = fa;
        }
    }
    __syncthreads();
    CKV_TMARK(41);
    const int cb = sh.cut_bin, above = sh.cut_above;
    if (cb < 0) {
        thr = 0ull;
        return true;
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (bin[j] == cb) {
            const int i = atomicAdd(&sh.ccount, 1);
            if (i < 64) {
                sh.ckey[i] = comm_key(sv[j], slab_id(tid, j));
                sh.csz[i] = w[j];
            }
        }
    }
    __syncthreads();
    CKV_TMARK(42);
    const int cnt = sh.ccount;
    if (cnt > 64) {
        __syncthreads();
        return false;
    }
    if (wave == 0) {
        // Each candidate of the cut bin sums the token weight of the better
        // ones; the cut is the best candidate whose inclusive weight overflows.
        const unsigned long long mine = lane < cnt ? sh.ckey[lane] : 0ull;
        const int msz = lane < cnt ? sh.csz[lane] : 0;
        int better = 0;
        for (int k0 = 0; k0 < cnt; k0 += 8) {  // k0 + 7 < 64: reads stay inside ckey/csz
            unsigned long long kk[8];
            int ss[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                kk[u] = sh.ckey[k0 + u];
                ss[u] = sh.csz[k0 + u];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < cnt && kk[u] > mine) better += ss[u];
        }
        const bool over = lane < cnt && above + better + msz > budget;
        const unsigned long long cut = wave_max_u64(over ? mine : 0ull);
        if (lane == 0) sh.thr = cut;
    }
    __syncthreads();
    thr = sh.thr;  // sh.thr is written once per kernel: no barrier needed after the read
    return true;
}

template <int NS>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
    constexpr int EPT = 4 * NS;
    __shared__ SelShared sh;
    const int g = p.g0 + blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    CKV_TMARK(10);
    const int C = p.c_cap;
    const int nc = min(p.n_comm[g], C);
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int L = p.seq_len[gc.b];
    const int ns = min(p.n_sinks, max(L, 0));
    const float *sc = p.scores + (size_t)g * C;
    const int32_t *sz = p.size + (size_t)g * C;
    const int32_t *offs = p.offs + (size_t)g * offs_stride(C);
    int32_t *tl = p.tok_list + (size_t)g * p.t_cap;

    // Sizes, scores and CSR offsets of this thread's four communities of every
    // slab, 16 bytes per load, and the tail entries.  c0 % 4 == 0 and C % 256
    // == 0, so a 16-byte load from c0 < C stays inside the row and offs[c0 + 4]
    // exists (the offsets row holds C + 4 entries).  Entries at or past n_comm
    // are masked after the loads.
    int s[EPT], o0[EPT], o1[EPT];
    float sv[EPT];
    {
        int4 s4[NS], o4[NS];
        float4 v4[NS];
        int on[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int c0 = j * kSlab + 4 * tid;
            s4[j] = make_int4(0, 0, 0, 0);
            o4[j] = make_int4(0, 0, 0, 0);
            v4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            on[j] = 0;
            if (c0 < C) {
                s4[j] = *reinterpret_cast<const int4 *>(sz + c0);
                v4[j] = *reinterpret_cast<const float4 *>(sc + c0);
                o4[j] = *reinterpret_cast<const int4 *>(offs + c0);
                on[j] = offs[c0 + 4];
            }
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int c0 = j * kSlab + 4 * tid;
            s[4 * j] = c0 < nc ? s4[j].x : 0;
            s[4 * j + 1] = c0 + 1 < nc ? s4[j].y : 0;
            s[4 * j + 2] = c0 + 2 < nc ? s4[j].z : 0;
            s[4 * j + 3] = c0 + 3 < nc ? s4[j].w : 0;
            sv[4 * j] = v4[j].x;
            sv[4 * j + 1] = v4[j].y;
            sv[4 * j + 2] = v4[j].z;
            sv[4 * j + 3] = v4[j].w;
            o0[4 * j] = o4[j].x;
            o0[4 * j + 1] = o4[j].y;
            o0[4 * j + 2] = o4[j].z;
            o0[4 * j + 3] = o4[j].w;
            o1[4 * j] = o4[j].y;
            o1[4 * j + 1] = o4[j].z;
            o1[4 * j + 2] = o4[j].w;
            o1[4 * j + 3] = on[j];
        }
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

    // LDS state the cut starts from, cleared under the first barrier below.
    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;
    sh.bw[tid] = 0;
    if (tid == 0) sh.ccount = 0;

    // Score range of the non-empty communities.
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (sv[j] == 0.f) sv[j] = 0.f;  // one key for +0 and -0
        if (s[j] > 0) {
            lo = fminf(lo, sv[j]);
            hi = fmaxf(hi, sv[j]);
        }
    }
    lo = wave_min_f(lo);
    hi = wave_max_f(hi);
    if (lane == 0) {
        sh.red_lo[wave] = lo;
        sh.red_hi[wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        lo = fminf(lo, sh.red_lo[i]);
        hi = fmaxf(hi, sh.red_hi[i]);
    }
    const bool any = hi >= lo;  // uniform: some community is non-empty
    // Best-ranked community: the lowest id among those scoring hi (read by
    // thread 0 at the end, after several barriers).
    uint32_t best = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
        if (s[j] > 0 && sv[j] == hi) best = min(best, (uint32_t)slab_id(tid, j));
    best = wave_min_u32(best);
    if (lane == 0) sh.red_id[wave] = best;
    CKV_TMARK(11);

    unsigned long long thr = ~0ull;  // nothing taken when there is no candidate
    if (any) {
        if (!value_cut<EPT>(sv, s, p.budget, lo, hi, sh, thr)) thr = radix_cut<EPT>(sv, s, false, p.budget, sh);
        if (p.max_comm > 0) thr = umax64(thr, radix_cut<EPT>(sv, s, true, p.max_comm, sh));
    }
    CKV_TMARK(12);

    // taken <=> key > thr, tested in 32-bit pieces
    const uint32_t thr_u = (uint32_t)(thr >> 32), thr_id = 0xFFFFFFFFu - (uint32_t)thr;
    bool taken[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const uint32_t u = ordered_bits(sv[j]), c = (uint32_t)slab_id(tid, j);
        taken[j] = s[j] > 0 && (u > thr_u || (u == thr_u && c < thr_id));
        if (taken[j]) atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    CKV_TMARK(43);
    // Per slab: taken communities and their base members; then taken tail entries.
    constexpr int NV = 2 * NS + 1;
    int v[NV], ex[NV], tot[NV];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        v[j] = 0;
        v[NS + j] = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (taken[4 * j + k]) {
                v[j] += 1;
                v[NS + j] += o1[4 * j + k] - o0[4 * j + k];
            }
        }
    }
    int f[kTailPerThread];
    v[2 * NS] = 0;
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
        const int i = tid * kTailPerThread + j;
        const int c = tcomm[j];
        f[j] = (i < tn && c >= 0 && c < C && ((sh.bits[c >> 5] >> (c & 31)) & 1u)) ? 1 : 0;
        v[2 * NS] += f[j];
    }
    block_scan_multi<kSelThreads, NV>(v, ex, tot, sh.scan);
    int nsel = 0, ntok = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        nsel += tot[j];
        ntok += tot[NS + j];
    }
    const int ntail = tot[2 * NS];
    CKV_TMARK(13);

    const int32_t *toks = p.toks + (size_t)g * p.l_cap;
    const bool lds_copy = nsel <= kSelLds;  // uniform
    {
        int kbase = 0, tbase = 0;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            int kpos = kbase + ex[j], rel = tbase + ex[NS + j];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = 4 * j + k;
                if (taken[e]) {
                    const int len = o1[e] - o0[e];
                    p.sel[(size_t)g * C + kpos] = slab_id(tid, e);
                    if (lds_copy) {
                        sh.soff[kpos] = o0[e];
                        sh.spref[kpos] = rel;
                    } else {
                        for (int i = 0; i < len; ++i) tl[ns + rel + i] = toks[o0[e] + i];
                    }
                    rel += len;
                    ++kpos;
                }
            }
            kbase += tot[j];
            tbase += tot[NS + j];
        }
    }
    for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
    // Taken tail members, in tail order, after the base members.
    {
        int tdst = ns + ntok + ex[2 * NS];
#pragma unroll
        for (int j = 0; j < kTailPerThread; ++j)
            if (f[j]) tl[tdst++] = tpos[j];
    }
    __syncthreads();
    CKV_TMARK(14);
    if (lds_copy) {
        // Slot j belongs to the last taken community whose first slot is <= j.
        for (int j0 = 0; j0 < ntok; j0 += 4 * kSelThreads) {
            int val[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                val[u] = 0;
                if (j < ntok) {
                    int a = 0, b = nsel - 1;
                    while (a < b) {
                        const int mid = (a + b + 1) >> 1;
                        if (sh.spref[mid] <= j) a = mid;
                        else b = mid - 1;
                    }
                    val[u] = toks[sh.soff[a] + (j - sh.spref[a])];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                if (j < ntok) tl[ns + j] = val[u];
            }
        }
    }
    CKV_TMARK(15);

    if (tid == 0) {
        uint32_t b = 0xFFFFFFFFu;
        for (int i = 0; i < kSelThreads / 64; ++i) b = min(b, sh.red_id[i]);
        p.sel_n[g] = nsel;
        p.tok_n[g] = ns + ntok + ntail;
        p.top[g] = any ? (int)b : -1;
    }
    CKV_TMARK(16);
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
    const Window w = window_of(idx);
    p.g0 = w.first;
    const int ns = ceil_div(idx->c_cap, kSlab);
    const dim3 grid(w.count), block(kSelThreads);
    if (ns <= 1) CKV_LAUNCH((select_kernel<1>), grid, block, s, p);
    else if (ns <= 2) CKV_LAUNCH((select_kernel<2>), grid, block, s, p);
    else if (ns <= 3) CKV_LAUNCH((select_kernel<3>), grid, block, s, p);
    else CKV_LAUNCH((select_kernel<4>), grid, block, s, p);
    return hipGetLastError();
}

}  // namespace ckv
