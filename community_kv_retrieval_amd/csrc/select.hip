// Budgeted community retrieval (the CommunityKV page, Figure 1 panel (3): the
// communities whose centroids score best are retrieved, and Tables 2-3 bound
// their tokens by a budget).
//
// One 1024-thread block per graph.  The communities are read in slabs of 4096:
// in slab j thread t owns communities 4096 j + 4 t .. 4096 j + 4 t + 3, so
// every 16-byte load of a wave covers 1 KB of consecutive memory.  A capacity
// at most 1024 past whole slabs adds one column instead of a fourth-empty
// slab: thread t also owns community 4096 NS + t (NS whole slabs).
// Communities rank by their exact score (float32 of the float64 product of
// the graph's query with the float32 centroid), higher first, ties to the
// lower id; as one number that is the 64-bit key (order-preserving bits of the
// score) << 32 | (~id).  The taken set is the longest prefix of the ranking
// that fits the budget, i.e. every key above the key of the first community
// that overflows it (the cut).
//
// The scores given are screening scores s~ with |s - s~| <= E (the scoring
// kernel's bound), i.e. every exact score lies in [L, U] = [s~ - E, s~ + E].
// Two token-weighted histograms over 1024 equal-width bins (a monotone map, so
// bins keep the order) of U and of L, each walked from the top, give the bin
// b_h where the U walk overflows the budget and the bin b_l where the L walk
// does.  Every community whose L bin is above b_h is certainly taken: all
// communities ranked above it have U at least as high, and those weigh no more
// than the budget.  Every community whose U bin is below b_l is certainly not:
// the communities whose L bin reaches b_l all rank above it and overflow the
// budget.  The communities in between (the band), and those whose U reaches
// the largest L (the candidates for the best community), get their exact
// score from the float32 centroid rows, one 16-lane group per community, and the
// band is cut with what the certain communities leave of the budget.  When the
// scores are degenerate, the band does not fit in LDS, or the community cap
// (max_comm) is set, every exact score is computed, slab by slab, and the cut
// is found on them directly: a histogram of the exact scores gives the bin
// holding the cut and the few communities of that bin are ranked exactly; a
// most-significant-digit radix select over the 64-bit keys, with
// token-weighted digit histograms, finds the same cut when that bin is
// crowded, and the community cap is the same radix select with unit weights.
//
// Then one block scan over per-slab (and per-column) counts gives every taken
// community its rank in ascending id order and its first slot in the token
// list, and every taken tail entry its slot after them.  The list is written as sinks, the base
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
// Communities whose exact score the screened path computes (band and
// best-community candidates); more than that switches to exact scores for all.
constexpr int kList = 2048;
constexpr uint32_t kBand = 1u << 30, kTopCand = 1u << 29;

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
    const float *cscale;
    const float *cent;  // float32 centroid rows (the exact scores' operand)
    const void *q;
    int bf16, D;
    int mode, Hq, Hkv, c_cap, l_cap, tail_cap, n_sinks, budget, max_comm, t_cap, g0;
    int32_t *sel;
    int32_t *sel_n;
    int32_t *top;
    int32_t *tok_list;
    int32_t *tok_n;
    CandArrays cand;  // from the scoring kernel (cand.ncand == 0: none)
    int cent_budget;  // centroid selection only
    int32_t *cent_sel;
    int32_t *cent_n;
};

struct SelShared {
    union __attribute__((aligned(16))) {
        struct {
            int soff[kSelLds];   // first base member in toks of the k-th taken community
            int spref[kSelLds];  // its first slot in the token list (after the sinks)
            __attribute__((aligned(16))) uint16_t owner[kSelLds];  // slot -> taken community (see copy_members)
        } cp;
        struct {
            unsigned long long key[kList];  // exact key
            int id[kList];                  // community | kBand | kTopCand
            int sz[kList];
        } ls;
        float exs[kSlab];  // exact scores of one slab
    } u;
    __attribute__((aligned(16))) int bw[kBins];   // token weight per bin: U (screened), exact score (exact path)
    __attribute__((aligned(16))) int bwl[kBins];  // token weight per bin of L
    uint32_t hw[256];  // radix select: token weight per digit
    uint32_t hn[256];  // radix select: candidates per digit
    uint32_t bits[CKV_MAX_C_CAP / 32];
    double qbar[128];  // interleaved for the exact scores: dimension l * (D / 16) + e at [e * 16 + l]
    float qabs[128];
    unsigned long long ckey[64];
    int csz[64];
    int ccount;
    int cut_bin, cut_above;
    int b_h, b_l;
    unsigned long long topkey, bandthr;
    int scan[(kSelThreads / 64) * 9];
    float red_lo[kSelThreads / 64], red_hi[kSelThreads / 64], red_lm[kSelThreads / 64];
    float red_ex[kSelThreads / 64];
    int wpre[CKV_MAX_C_CAP / 32];  // taken communities in the bit words before each word
    uint32_t red_id[kSelThreads / 64];
    unsigned long long prefix, mask, thr;
    long long rem;
    int done;
};

__device__ __forceinline__ unsigned long long comm_key(float s, int c) {
    if (s == 0.f) s = 0.f;  // one key for +0 and -0
    return ((unsigned long long)ordered_bits(s) << 32) | (0xFFFFFFFFu - (uint32_t)c);
}

// The float32 score a key was made from.
__device__ __forceinline__ float key_score(unsigned long long k) {
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Community of element e of thread tid: elements 0 .. 4 NS - 1 are four
// consecutive communities in each slab of 4096 (slab e / 4); the elements
// after them are single communities NS * 4096 + x * 1024 + tid (x = e - 4 NS),
// which cover a capacity just past a whole number of slabs.
template <int NS>
__device__ __forceinline__ int slab_id(int tid, int e) {
    return e < 4 * NS ? (e >> 2) * kSlab + 4 * tid + (e & 3) : NS * kSlab + (e - 4 * NS) * kSelThreads + tid;
}

// Block-wide exclusive prefix sums of NV ints per thread, in thread order, and
// their totals.  One barrier (LDS only: loads in flight keep flowing): every
// wave scans the wave totals itself.  `scratch` holds NT/64 * NV ints; the
// caller puts a barrier between two uses.
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
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int t = lane < NW ? scratch[lane * NV + k] : 0;
        const int ti = wave_incl_scan(t);
        tot[k] = __builtin_amdgcn_readlane(ti, NW - 1);
        const int before = wave > 0 ? __builtin_amdgcn_readlane(ti, wave > 0 ? wave - 1 : 0) : 0;
        ex[k] = before + x[k] - v[k];
    }
}

// Threshold key of a budget cut by radix select over 64-bit keys (0 = no
// candidate): the taken keys are those > threshold (0 = everything fits).
// `unit` counts candidates instead of their token weight (the community cap).
template <int N>
__device__ unsigned long long radix_cut(const unsigned long long (&key)[N], const int (&w)[N], bool unit,
                                        long long budget, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int j = 0; j < N; ++j) {
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
    if (kmax == 0ull) return 0ull;  // uniform: no candidate
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
        for (int j = 0; j < N; ++j) {
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

// Keys of this thread's communities (0 for empty ones).
template <int NS, int EPT>
__device__ __forceinline__ void comm_keys(const float (&sv)[EPT], const int (&w)[EPT],
                                          unsigned long long (&key)[EPT]) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = w[j] > 0 ? comm_key(sv[j], slab_id<NS>(threadIdx.x, j)) : 0ull;
}

// Budget cut through equal-width score bins (see the file comment).  The bin
// weights and the candidate count must be zero on entry.  Returns false,
// uniformly across the block, when the radix select has to decide.
template <int EPT, typename IdF>
__device__ bool value_cut(const float (&sv)[EPT], const int (&w)[EPT], int budget, float lo, float hi,
                          SelShared &sh, unsigned long long &thr, IdF idf) {
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
                sh.ckey[i] = comm_key(sv[j], idf(j));
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

// Exact score of n communities, one 16-lane group per community, stride 64
// groups: float32 of the float64 sum over d of qbar_d * cent[c][d], the
// float32 centroid row exactly as the index stores it (float32(csum / size)).
// The communities are the list entries (to_list) or the ids slab * 4096 + i of
// one slab (or of the column past the last whole slab, i < 1024).  Every lane
// loads its D/16 consecutive floats with 16-byte loads; the rows of four
// communities per group are in flight together.
template <int D>
__device__ __forceinline__ void exact_scores(const SelectParams &p, int g, int n, SelShared &sh,
                                             bool to_list, int slab) {
    constexpr int E = D / 16;  // floats per lane
    constexpr int R = 4;       // rows per group in flight
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const int nc = min(p.n_comm[g], p.c_cap);
    for (int i0 = grp; i0 < n; i0 += R * 64) {
        int cc[R], nn[R];
        float cs[R][E];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + 64 * r;
            const bool ok = i < n;
            if (to_list) {
                cc[r] = ok ? (sh.u.ls.id[i] & 0xFFFF) : 0;
                nn[r] = ok ? sh.u.ls.sz[i] : 0;
            } else {
                cc[r] = slab * kSlab + (ok ? i : 0);
                nn[r] = ok && cc[r] < nc ? p.size[(size_t)g * p.c_cap + cc[r]] : 0;
                if (cc[r] >= p.c_cap) cc[r] = 0;
            }
            const float *row = p.cent + ((size_t)g * p.c_cap + cc[r]) * D + l16 * E;
#pragma unroll
            for (int e = 0; e < E; e += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(row + e);
                cs[r][e] = f.x;
                cs[r][e + 1] = f.y;
                cs[r][e + 2] = f.z;
                cs[r][e + 3] = f.w;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double part = 0.0;
            if (nn[r] > 0) {
#pragma unroll
                for (int e = 0; e < E; ++e) part = fma(sh.qbar[e * 16 + l16], (double)cs[r][e], part);
            }
            const double S = row16_sum_d(part);
            const int i = i0 + 64 * r;
            if (l16 == 0 && i < n) {
                if (to_list) sh.u.ls.key[i] = comm_key((float)S, cc[r]);
                else sh.u.exs[i] = nn[r] > 0 ? (float)S : kNegInf;
            }
        }
    }
}

// The graph's query into sh.qbar (its head's q, or the sum of its group's q,
// exact in float64) and |float32(qbar)| into sh.qabs.  The (at most 8) heads
// are loaded unconditionally at clamped addresses, so they share the round
// trip of the loads issued before; the caller's barrier publishes the values.
__device__ __forceinline__ void load_qbar(const SelectParams &p, const GraphCoords &gc, SelShared &sh) {
    const int tid = threadIdx.x;
    constexpr int kMaxHeads = 8;
    float qv[kMaxHeads];
    const size_t q0 = ((size_t)gc.b * p.Hq + gc.qh0) * p.D + min(tid, p.D - 1);
    if (p.bf16) {
        const bf16_t *qb = reinterpret_cast<const bf16_t *>(p.q) + q0;
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h) qv[h] = to_f32(qb[(size_t)min(h, gc.nh - 1) * p.D]);
    } else {
        const float *qf = reinterpret_cast<const float *>(p.q) + q0;
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h) qv[h] = qf[(size_t)min(h, gc.nh - 1) * p.D];
    }
    if (tid < p.D) {
        double a = 0.0;
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h)
            if (h < gc.nh) a += (double)qv[h];
        // dimension d = 16-lane group lane l * (D / 16) + e at [e][l]: the
        // exact scores' reads of one e by 16 lanes are 128 contiguous bytes
        sh.qbar[(tid % (p.D / 16)) * 16 + tid / (p.D / 16)] = a;
        sh.qabs[tid] = fabsf((float)a);
    }
}

// Wave-wide inclusive max of non-negative ints (the DPP steps of
// wave_incl_scan with max for the sum; lanes shifted in from outside a row
// contribute 0).
__device__ __forceinline__ int wave_incl_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));  // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));  // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));  // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));  // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return x;
}

// Base members of the nsel taken communities into the token list after the
// ns sinks: taken community r (rank order) owns slots sh.u.cp.spref[r] up to
// the next community's first slot and copies toks[soff[r] + j - spref[r]]
// into slot j.  For lists of up to kSelLds slots the owner of every slot comes
// from one block-wide max-scan: each community with members marks its first
// slot with its rank in sh.u.cp.owner (zero elsewhere), and a slot's owner is
// the largest mark at or before it.  Thread t handles slots 4t .. 4t + 3.
// Longer lists find each slot's owner by binary lifting over spref.  Starts
// and ends with the caller's barrier (spref and soff complete).
__device__ __forceinline__ void copy_members(const int32_t *toks, int32_t *tl, int ns, int nsel, int ntok,
                                             SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (ntok <= kSelLds) {  // uniform
        *reinterpret_cast<uint2 *>(&sh.u.cp.owner[4 * tid]) = make_uint2(0u, 0u);
        lds_barrier();
        for (int r = tid; r < nsel; r += kSelThreads) {
            const int s0 = sh.u.cp.spref[r];
            const int s1 = r + 1 < nsel ? sh.u.cp.spref[r + 1] : ntok;
            if (s1 > s0) sh.u.cp.owner[s0] = (uint16_t)r;
        }
        lds_barrier();
        const uint2 ow = *reinterpret_cast<const uint2 *>(&sh.u.cp.owner[4 * tid]);
        int m[4] = {(int)(ow.x & 0xFFFFu), (int)(ow.x >> 16), (int)(ow.y & 0xFFFFu), (int)(ow.y >> 16)};
        m[1] = max(m[1], m[0]);
        m[2] = max(m[2], m[1]);
        m[3] = max(m[3], m[2]);
        // ranks marked before this thread's slots
        const int incl = wave_incl_max(m[3]);
        int before = __shfl_up(incl, 1, 64);
        if (lane == 0) before = 0;
        if (lane == 63) sh.scan[wave] = incl;
        lds_barrier();
        for (int w = 0; w < wave; ++w) before = max(before, sh.scan[w]);
        int val[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * tid + u, r = max(before, m[u]);
            val[u] = j < ntok ? toks[sh.u.cp.soff[r] + (j - sh.u.cp.spref[r])] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (4 * tid + u < ntok) tl[ns + 4 * tid + u] = val[u];
        return;
    }
    const int top_step = nsel > 1 ? 1 << (31 - __builtin_clz(nsel - 1)) : 0;  // uniform
    for (int j0 = 0; j0 < ntok; j0 += 4 * kSelThreads) {
        int val[4], at[4] = {0, 0, 0, 0};
        for (int step = top_step; step > 0; step >>= 1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                const int nx = at[u] + step;
                if (nx < nsel && sh.u.cp.spref[nx] <= j) at[u] = nx;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u * kSelThreads + tid;
            val[u] = j < ntok ? toks[sh.u.cp.soff[at[u]] + (j - sh.u.cp.spref[at[u]])] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u * kSelThreads + tid;
            if (j < ntok) tl[ns + j] = val[u];
        }
    }
}

// Exact scores of the nlist entries of the list (band members, flagged
// kBand, and best-community candidates, flagged kTopCand), the best community
// into sh.topkey, and the cut of the nband band members with what the certain
// communities leave of the budget (rest): band members above the cut get
// their bit in sh.bits.  The list is in sh.u.ls, written before a barrier.
template <int D>
__device__ void list_cut(const SelectParams &p, int g, int nlist, int nband, int rest, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    exact_scores<D>(p, g, nlist, sh, true, 0);
    sh.bw[tid] = 0;  // the band cut starts from empty bins
    if (tid == 0) sh.ccount = 0;
    lds_barrier();
    CKV_TMARK(55);
    if (nlist <= 64) {  // uniform: the usual case, finished by wave 0
        if (wave == 0) {
            // best community, and each band member sums the weight of the
            // better ones; the cut is the best member whose inclusive
            // weight overflows what the certain communities leave
            const bool ok = lane < nlist;
            const int id = ok ? sh.u.ls.id[lane] : 0;
            const unsigned long long key = ok ? sh.u.ls.key[lane] : 0ull;
            const int sz = ok ? sh.u.ls.sz[lane] : 0;
            const bool band = (id & kBand) != 0;
            const unsigned long long tk = wave_max_u64((id & kTopCand) ? key : 0ull);
            long long better = 0;
            for (int k0 = 0; k0 < nlist; k0 += 8) {  // k0 + 7 < 64 <= kList
                unsigned long long kk[8];
                int ii[8], ss[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    kk[u] = sh.u.ls.key[k0 + u];
                    ii[u] = sh.u.ls.id[k0 + u];
                    ss[u] = sh.u.ls.sz[k0 + u];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (k0 + u < nlist && (ii[u] & kBand) && kk[u] > key) better += ss[u];
            }
            const bool over = band && better + sz > rest;
            const unsigned long long cut = wave_max_u64(over ? key : 0ull);
            if (band && key > cut) {
                const int c = id & 0xFFFF;
                atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
            }
            if (lane == 0 && tk) sh.topkey = tk;
        }
        // the barrier before the taken flags are read orders these writes
    } else {
        // Best community: the largest exact key among the candidates; the
        // band entries with their exact scores and the band's score range.
        constexpr int NB = kList / kSelThreads;
        unsigned long long bk[NB], tk = 0ull;
        int bwt[NB];
        float bs[NB], blo = __builtin_huge_valf(), bhi = -__builtin_huge_valf();
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int i = tid + r * kSelThreads;
            const int id = i < nlist ? sh.u.ls.id[i] : 0;
            const unsigned long long key = i < nlist ? sh.u.ls.key[i] : 0ull;
            if (id & kTopCand) tk = umax64(tk, key);
            const bool band = (id & kBand) != 0;
            bk[r] = band ? key : 0ull;
            bwt[r] = band ? sh.u.ls.sz[i] : 0;
            bs[r] = band ? key_score(key) : 0.f;
            if (band) {
                blo = fminf(blo, bs[r]);
                bhi = fmaxf(bhi, bs[r]);
            }
        }
        tk = wave_max_u64(tk);
        blo = wave_min_f(blo);
        bhi = wave_max_f(bhi);
        if (lane == 0) {
            if (tk) atomicMax(&sh.topkey, tk);
            sh.red_lo[wave] = blo;
            sh.red_hi[wave] = bhi;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSelThreads / 64; ++i) {
            blo = fminf(blo, sh.red_lo[i]);
            bhi = fmaxf(bhi, sh.red_hi[i]);
        }
        // Cut of the band with the budget the certain communities leave.
        unsigned long long bthr = 0ull;
        if (nband > 0 && nband <= 64) {
            // few band members: wave 0 compacts them into ckey/csz and each
            // one sums the weight of the better ones; the cut is the best
            // member whose inclusive weight overflows what is left
            if (wave == 0) {
                int got = 0;
                for (int i0 = 0; i0 < nlist; i0 += 64) {
                    const int i = i0 + lane;
                    const bool b = i < nlist && (sh.u.ls.id[i] & kBand);
                    const unsigned long long m = __ballot(b);
                    if (b) {
                        const int at = got + __popcll(m & ((1ull << lane) - 1ull));
                        sh.ckey[at] = sh.u.ls.key[i];
                        sh.csz[at] = sh.u.ls.sz[i];
                    }
                    got += __popcll(m);
                }
                const unsigned long long mine = lane < nband ? sh.ckey[lane] : 0ull;
                const int msz = lane < nband ? sh.csz[lane] : 0;
                long long better = 0;
                for (int k0 = 0; k0 < nband; k0 += 8) {  // k0 + 7 < 64: inside ckey/csz
                    unsigned long long kk[8];
                    int ss[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        kk[u] = sh.ckey[k0 + u];
                        ss[u] = sh.csz[k0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (k0 + u < nband && kk[u] > mine) better += ss[u];
                }
                const bool over = lane < nband && better + msz > rest;
                const unsigned long long cut = wave_max_u64(over ? mine : 0ull);
                if (lane == 0) sh.bandthr = cut;
            }
            __syncthreads();
            bthr = sh.bandthr;
        } else if (nband > 64) {  // uniform
            if (!value_cut<NB>(bs, bwt, rest, blo, bhi, sh, bthr,
                               [&](int r) { return (int)(0xFFFFFFFFu - (uint32_t)bk[r]); }))
                bthr = radix_cut<NB>(bk, bwt, false, rest, sh);
        }
        // band members above the band cut are taken: marked from the list side
        for (int i = tid; i < nlist; i += kSelThreads) {
            const int id = sh.u.ls.id[i];
            if ((id & kBand) && sh.u.ls.key[i] > bthr) {
                const int c = id & 0xFFFF;
                atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
            }
        }
    }
}

// The U walk (wave 0: bins bw) and the L walk (wave 1: bw + bwl) from the
// top bin down: sh.b_h and sh.b_l become the bins where the running token
// weight first exceeds the budget (-1: it never does).  Lane l owns the 16
// bins below kBins - 16 l; a prefix over the lanes gives each lane the weight
// above its bins.  The caller's barrier publishes the result.
__device__ __forceinline__ void walk_bins(int budget, SelShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (wave >= 2) return;
    // the lane's 16 bins as four 16-byte reads (v[k]: bin kBins - 1 - 16 lane - k)
    const int base = kBins - 16 * (lane + 1);
    int v[16], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int4 a = *reinterpret_cast<const int4 *>(&sh.bw[base + 4 * i]);
        if (wave == 1) {
            const int4 c = *reinterpret_cast<const int4 *>(&sh.bwl[base + 4 * i]);
            a.x += c.x;
            a.y += c.y;
            a.z += c.z;
            a.w += c.w;
        }
        v[15 - 4 * i] = a.x;
        v[14 - 4 * i] = a.y;
        v[13 - 4 * i] = a.z;
        v[12 - 4 * i] = a.w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) tot += v[k];
    const int incl = wave_incl_scan(tot);
    int acc = incl - tot, found = -1;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if (found < 0 && acc + v[k] > budget) found = kBins - 1 - (lane * 16 + k);
        acc += v[k];
    }
    const unsigned long long bal = __ballot(found >= 0);
    const int src = bal ? __ffsll((long long)bal) - 1 : 0;
    const int fb = __shfl(found, src, 64);
    if (lane == 0) {
        if (wave == 0) sh.b_h = bal ? fb : -1;
        else sh.b_l = bal ? fb : -1;
    }
}

// Candidate path.  The scoring kernel gave, of every wave of 64 communities,
// the kCandPerWave of largest upper bound U and the largest U it left out
// (EX).  The histograms, walks, classification and band cut above run on the
// candidates only.  Every community the cut can depend on has its U in a bin
// at or above b_l (the bin where the L walk overflows the budget): taken,
// band and best-community candidates alike.  So when the largest left-out U
// bins below b_l, the candidates hold all of them and the result is that of
// every community.  Otherwise (or when the L walk does not overflow, the range
// is degenerate or the list is too long) this returns false, uniformly, and
// the caller runs the path over every community.  On success it has written
// sel, the sinks and the taken tail members, and left the taken communities'
// first slots and members in sh.u.cp for the member copy; the counts come back
// in nsel_out (taken communities), ntok_out (their base members) and
// ntail_out (taken tail members).
template <int NC, int D>
__device__ bool select_from_candidates(const SelectParams &p, int g, const GraphCoords &gc, int ns,
                                       SelShared &sh, int &nsel_out, int &ntok_out, int &ntail_out) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = p.c_cap, ncand = p.cand.ncand;
    const size_t cb = (size_t)g * ncand;
    int cid[NC], csz[NC], co0[NC], clen[NC];
    float cu[NC], cl[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int i = tid + j * kSelThreads;
        const size_t k = cb + (i < ncand ? i : 0);
        cid[j] = i < ncand ? p.cand.id[k] : -1;
        cu[j] = p.cand.u[k];
        cl[j] = p.cand.l[k];
        csz[j] = p.cand.sz[k];
        co0[j] = p.cand.o0[k];
        clen[j] = p.cand.len[k];
    }
    const int nex = ncand / kCandPerWave;
    float exv = tid < nex ? p.cand.ex[(size_t)g * nex + tid] : kNegInf;
    const int tn = p.tail_len[g];
    int tcomm[kTailPerThread], tpos[kTailPerThread];
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
        const int i = tid * kTailPerThread + j;
        const bool in = i < p.tail_cap;
        tcomm[j] = in ? p.tail_comm[(size_t)g * p.tail_cap + i] : -1;
        tpos[j] = in ? p.tail_pos[(size_t)g * p.tail_cap + i] : 0;
    }
    load_qbar(p, gc, sh);
    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;
    sh.bw[tid] = 0;
    sh.bwl[tid] = 0;
    if (tid == 0) {
        sh.ccount = 0;
        sh.topkey = 0ull;
    }
    // range of the candidates' bounds, the largest L, and EX
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf(), lmax = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if (cid[j] >= 0) {
            lo = fminf(lo, cl[j]);
            hi = fmaxf(hi, cu[j]);
            lmax = fmaxf(lmax, cl[j]);
        }
    }
    lo = wave_min_f(lo);
    hi = wave_max_f(hi);
    lmax = wave_max_f(lmax);
    exv = wave_max_f(exv);
    if (lane == 0) {
        sh.red_lo[wave] = lo;
        sh.red_hi[wave] = hi;
        sh.red_lm[wave] = lmax;
        sh.red_ex[wave] = exv;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        lo = fminf(lo, sh.red_lo[i]);
        hi = fmaxf(hi, sh.red_hi[i]);
        lmax = fmaxf(lmax, sh.red_lm[i]);
        exv = fmaxf(exv, sh.red_ex[i]);
    }
    const float bscale = (float)kBins / (hi - lo);
    if (!(hi > lo) || !(bscale < __builtin_huge_valf())) {  // uniform
        CKV_TCOUNT(60);
        __syncthreads();
        return false;
    }
    CKV_TMARK(11);
    // token-weighted histograms of U (bw) and of L (bw + corrections in bwl)
    int bb[NC];
    uint32_t tcm = 0u;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        bb[j] = 0;
        if (cid[j] >= 0) {
            const int bu = min(kBins - 1, (int)((cu[j] - lo) * bscale));
            const int bl = min(kBins - 1, (int)((cl[j] - lo) * bscale));
            bb[j] = (bu << 16) | bl;
            atomicAdd(&sh.bw[bu], csz[j]);
            if (bl != bu) {
                atomicAdd(&sh.bwl[bl], csz[j]);
                atomicSub(&sh.bwl[bu], csz[j]);
            }
            if (cu[j] >= lmax) tcm |= 1u << j;
        }
    }
    __syncthreads();
    CKV_TMARK(50);
    walk_bins(p.budget, sh);
    __syncthreads();
    CKV_TMARK(51);
    const int b_h = sh.b_h, b_l = sh.b_l;
    const int bex = exv < lo ? -1 : min(kBins - 1, (int)((exv - lo) * bscale));
    if (b_l < 0 || bex >= b_l) {  // uniform: a left-out community may matter
        CKV_TCOUNT(61);
        __syncthreads();
        return false;
    }
    uint32_t cert = 0u, wantm = 0u, bandm = 0u;
    int v[3] = {0, 0, 0}, ex[3], tot[3];  // list entries, band entries, certain weight
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        if (cid[j] < 0) continue;
        const bool ce = (bb[j] & 0xFFFF) > b_h;
        const bool band = !ce && (bb[j] >> 16) >= b_l;
        const bool tc = (tcm >> j) & 1u;
        if (ce) {
            cert |= 1u << j;
            v[2] += csz[j];
        }
        if (band) {
            bandm |= 1u << j;
            v[1] += 1;
        }
        if (band || tc) {
            wantm |= 1u << j;
            v[0] += 1;
        }
    }
    block_scan_multi<kSelThreads, 3>(v, ex, tot, sh.scan);
    const int nlist = tot[0];
    if (nlist > kList) {  // uniform
        CKV_TCOUNT(62);
        __syncthreads();
        return false;
    }
    {
        int i = ex[0];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            if ((wantm >> j) & 1u) {
                sh.u.ls.id[i] = cid[j] | (((bandm >> j) & 1u) ? (int)kBand : 0) |
                                (((tcm >> j) & 1u) ? (int)kTopCand : 0);
                sh.u.ls.sz[i] = csz[j];
                ++i;
            }
        }
    }
    CKV_TMARK(52);
    lds_barrier();
    list_cut<D>(p, g, nlist, tot[1], p.budget - tot[2], sh);
#pragma unroll
    for (int j = 0; j < NC; ++j)
        if ((cert >> j) & 1u) atomicOr(&sh.bits[cid[j] >> 5], 1u << (cid[j] & 31));
    lds_barrier();
    CKV_TMARK(12);

    // Taken ids in ascending order: each bit word's rank offset, and the taken
    // tail entries' places.
    const int W = C / 32;
    const uint32_t myw = tid < W ? sh.bits[tid] : 0u;
    int f[kTailPerThread];
    int v2[2] = {(int)__popc(myw), 0}, ex2[2], tot2[2];
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
        const int i = tid * kTailPerThread + j;
        const int c = tcomm[j];
        f[j] = (i < tn && c >= 0 && c < C && ((sh.bits[c >> 5] >> (c & 31)) & 1u)) ? 1 : 0;
        v2[1] += f[j];
    }
    block_scan_multi<kSelThreads, 2>(v2, ex2, tot2, sh.scan);
    if (tid < W) sh.wpre[tid] = ex2[0];
    const int nsel = tot2[0], ntail = tot2[1];
    lds_barrier();
    CKV_TMARK(43);
    // every taken candidate at its rank: the selection, its first base member
    // and (for now) its base-member count
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = cid[j];
        if (c < 0) continue;
        const uint32_t wd = sh.bits[c >> 5];
        if ((wd >> (c & 31)) & 1u) {
            const int r = sh.wpre[c >> 5] + __popc(wd & ((1u << (c & 31)) - 1u));
            p.sel[(size_t)g * C + r] = c;
            sh.u.cp.soff[r] = co0[j];
            sh.u.cp.spref[r] = clen[j];
        }
    }
    lds_barrier();
    // first slot of every taken community: exclusive scan of the counts in rank
    // order, four ranks per thread
    int lenv[4], lsum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = tid * 4 + k;
        lenv[k] = r < nsel ? sh.u.cp.spref[r] : 0;
        lsum += lenv[k];
    }
    int v3[1] = {lsum}, ex3[1], tot3[1];
    block_scan_multi<kSelThreads, 1>(v3, ex3, tot3, sh.scan);
    {
        int run = ex3[0];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = tid * 4 + k;
            if (r < nsel) sh.u.cp.spref[r] = run;
            run += lenv[k];
        }
    }
    const int ntok = tot3[0];
    CKV_TMARK(13);
    int32_t *tl = p.tok_list + (size_t)g * p.t_cap;
    for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
    {
        int tdst = ns + ntok + ex2[1];
#pragma unroll
        for (int j = 0; j < kTailPerThread; ++j)
            if (f[j]) tl[tdst++] = tpos[j];
    }
    nsel_out = nsel;
    ntok_out = ntok;
    ntail_out = ntail;
    return true;  // the caller's barrier publishes spref / soff for the member copy
}

template <int NS, int X, int NC, int D>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
    constexpr int EPT = 4 * NS + X;
    constexpr int NGR = NS + X;  // id-ordered groups: the slabs, then the single columns
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
    const float *scl = p.cscale + (size_t)g * C;
    int32_t *tl = p.tok_list + (size_t)g * p.t_cap;
    int nsel = 0, ntok = 0, ntail = 0;
    bool lds_copy = true, any = true;
    bool done = false;
    if (p.max_comm == 0 && p.cand.ncand > 0)  // uniform
        done = select_from_candidates<NC, D>(p, g, gc, ns, sh, nsel, ntok, ntail);
    if (!done) {

        // Sizes, screening scores, scales and CSR offsets of this thread's four
        // communities of every slab, 16 bytes per load, and the tail entries.
        // c0 % 4 == 0 and C % 256 == 0, so a 16-byte load from c0 < C stays inside
        // the row and offs[c0 + 4] exists (the offsets row holds C + 4 entries).
        // Entries at or past n_comm are masked after the loads.
        int s[EPT], o0[EPT], on[NS];
        float sv[EPT], se[EPT];
        {
            int4 s4[NS], o4[NS];
            float4 v4[NS], e4[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const int c0 = j * kSlab + 4 * tid;
                s4[j] = make_int4(0, 0, 0, 0);
                o4[j] = make_int4(0, 0, 0, 0);
                v4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                e4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                on[j] = 0;
                if (c0 < C) {
                    s4[j] = *reinterpret_cast<const int4 *>(sz + c0);
                    v4[j] = *reinterpret_cast<const float4 *>(sc + c0);
                    e4[j] = *reinterpret_cast<const float4 *>(scl + c0);
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
                se[4 * j] = e4[j].x;
                se[4 * j + 1] = e4[j].y;
                se[4 * j + 2] = e4[j].z;
                se[4 * j + 3] = e4[j].w;
                o0[4 * j] = o4[j].x;
                o0[4 * j + 1] = o4[j].y;
                o0[4 * j + 2] = o4[j].z;
                o0[4 * j + 3] = o4[j].w;
            }
        }
        // The single columns past the slabs: one community each, 4-byte loads, and
        // the next community's offset for the end of its base members.
        int onx[X > 0 ? X : 1];
#pragma unroll
        for (int x = 0; x < X; ++x) {
            const int c = NS * kSlab + x * kSelThreads + tid, e = 4 * NS + x;
            const bool in = c < C;
            const int sz_c = in ? sz[c] : 0;
            sv[e] = in ? sc[c] : 0.f;
            se[e] = in ? scl[c] : 0.f;
            o0[e] = in ? offs[c] : 0;
            onx[x] = in ? offs[c + 1] : 0;
            s[e] = c < nc ? sz_c : 0;
        }
        // end of the base members of element e: the next element's start
        auto o1 = [&](int e) { return e >= 4 * NS ? onx[e - 4 * NS] : (e & 3) == 3 ? on[e >> 2] : o0[e + 1]; };
        const int tn = p.tail_len[g];
        int tcomm[kTailPerThread], tpos[kTailPerThread];
#pragma unroll
        for (int j = 0; j < kTailPerThread; ++j) {
            const int i = tid * kTailPerThread + j;
            const bool in = i < p.tail_cap;
            tcomm[j] = in ? p.tail_comm[(size_t)g * p.tail_cap + i] : -1;
            tpos[j] = in ? p.tail_pos[(size_t)g * p.tail_cap + i] : 0;
        }
        // The graph's query, loaded with the loads above.
        load_qbar(p, gc, sh);

        // LDS state the cuts start from, cleared under the first barrier below.
        for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;
        sh.bw[tid] = 0;
        sh.bwl[tid] = 0;
        if (tid == 0) {
            sh.ccount = 0;
            sh.topkey = 0ull;
        }
        __syncthreads();

        // Interval [L, U] of every exact score: E = cscale * |qbar|_1 * kScreenK
        // plus 2^-20 |s~| for the float32 roundings of s~, of the exact score and
        // of U and L themselves.
        float qn = sh.qabs[lane] * (lane < p.D ? 1.f : 0.f);
        if (lane + 64 < p.D) qn += sh.qabs[lane + 64];
        const float kq = wave_sum_f(qn) * kScreenK;
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf(), lmax = -__builtin_huge_valf();
        auto bound = [&](int j) { return screen_bound(sv[j], se[j], kq); };
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (s[j] > 0) {
                const float e = bound(j);
                lo = fminf(lo, sv[j] - e);
                hi = fmaxf(hi, sv[j] + e);
                lmax = fmaxf(lmax, sv[j] - e);
            }
        }
        lo = wave_min_f(lo);
        hi = wave_max_f(hi);
        lmax = wave_max_f(lmax);
        if (lane == 0) {
            sh.red_lo[wave] = lo;
            sh.red_hi[wave] = hi;
            sh.red_lm[wave] = lmax;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSelThreads / 64; ++i) {
            lo = fminf(lo, sh.red_lo[i]);
            hi = fmaxf(hi, sh.red_hi[i]);
            lmax = fmaxf(lmax, sh.red_lm[i]);
        }
        any = hi >= lo;  // uniform: some community is non-empty
        const float bscale = (float)kBins / (hi - lo);
        bool exact_all = p.max_comm > 0 || !(hi > lo) || !(bscale < __builtin_huge_valf());  // uniform
        CKV_TMARK(11);

        unsigned long long thr = ~0ull;  // nothing taken when there is no candidate
        uint32_t cert = 0u;  // bit j: community j of this thread is taken
        if (any && !exact_all) {
            // Token-weighted histograms of U (bw) and of L (bw + the corrections
            // in bwl of the few communities whose L falls in a lower bin); the U
            // walk overflows the budget in bin b_h, the L walk in bin b_l (-1: no
            // overflow).
            int bb[EPT];        // U bin << 16 | L bin
            uint32_t tcm = 0u;  // bit j: candidate for the best community
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const float e = bound(j), u = sv[j] + e, l = sv[j] - e;
                const int bu = min(kBins - 1, (int)((u - lo) * bscale));
                const int bl = min(kBins - 1, (int)((l - lo) * bscale));
                bb[j] = (bu << 16) | bl;
                if (s[j] > 0) {
                    atomicAdd(&sh.bw[bu], s[j]);
                    if (bl != bu) {  // rare: the L histogram differs from the U one
                        atomicAdd(&sh.bwl[bl], s[j]);
                        atomicSub(&sh.bwl[bu], s[j]);
                    }
                    if (u >= lmax) tcm |= 1u << j;
                }
            }
            __syncthreads();
            CKV_TMARK(50);
            walk_bins(p.budget, sh);
            __syncthreads();
            CKV_TMARK(51);
            const int b_h = sh.b_h, b_l = sh.b_l;
            // Certain, band and best-community candidates; the latter two go to the
            // list, at places a block scan of the per-thread counts assigns.
            uint32_t wantm = 0u, bandm = 0u;
            int v[3] = {0, 0, 0}, ex[3], tot[3];  // list entries, band entries, certain weight
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                if (s[j] <= 0) continue;
                const bool ce = (bb[j] & 0xFFFF) > b_h;
                const bool band = !ce && (bb[j] >> 16) >= b_l;
                const bool tc = (tcm >> j) & 1u;
                if (ce) {
                    cert |= 1u << j;
                    v[2] += s[j];
                }
                if (band) {
                    bandm |= 1u << j;
                    v[1] += 1;
                }
                if (band || tc) {
                    wantm |= 1u << j;
                    v[0] += 1;
                }
            }
            block_scan_multi<kSelThreads, 3>(v, ex, tot, sh.scan);
            CKV_TMARK(52);
            const int nlist = tot[0];
            if (nlist > kList) {
                exact_all = true;  // uniform
            } else {
                int i = ex[0];
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    if ((wantm >> j) & 1u) {
                        sh.u.ls.id[i] = slab_id<NS>(tid, j) | (((bandm >> j) & 1u) ? (int)kBand : 0) |
                                        (((tcm >> j) & 1u) ? (int)kTopCand : 0);
                        sh.u.ls.sz[i] = s[j];
                        ++i;
                    }
                }
                CKV_TMARK(53);
                __syncthreads();
                CKV_TMARK(54);
                list_cut<D>(p, g, nlist, tot[1], p.budget - tot[2], sh);
                CKV_TMARK(56);
            }
        }
        if (any && exact_all) {
            // Exact scores of every community, one slab at a time, then the cut on them.
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                __syncthreads();
                exact_scores<D>(p, g, min(kSlab, C - j * kSlab), sh, false, j);
                __syncthreads();
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e = 4 * j + k;
                    if (4 * tid + k < kSlab && j * kSlab + 4 * tid + k < C) sv[e] = sh.u.exs[4 * tid + k];
                }
            }
            if constexpr (X > 0) {
                __syncthreads();
                exact_scores<D>(p, g, max(0, min(X * kSelThreads, C - NS * kSlab)), sh, false, NS);
                __syncthreads();
#pragma unroll
                for (int x = 0; x < X; ++x)
                    if (NS * kSlab + x * kSelThreads + tid < C) sv[4 * NS + x] = sh.u.exs[x * kSelThreads + tid];
            }
            // exact range and best community
            float elo = __builtin_huge_valf(), ehi = -__builtin_huge_valf();
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                if (s[j] > 0) {
                    elo = fminf(elo, sv[j]);
                    ehi = fmaxf(ehi, sv[j]);
                }
            }
            elo = wave_min_f(elo);
            ehi = wave_max_f(ehi);
            __syncthreads();
            sh.bw[tid] = 0;
            if (tid == 0) sh.ccount = 0;
            if (lane == 0) {
                sh.red_lo[wave] = elo;
                sh.red_hi[wave] = ehi;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kSelThreads / 64; ++i) {
                elo = fminf(elo, sh.red_lo[i]);
                ehi = fmaxf(ehi, sh.red_hi[i]);
            }
            unsigned long long bk = 0ull;
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (s[j] > 0) bk = umax64(bk, comm_key(sv[j], slab_id<NS>(tid, j)));
            bk = wave_max_u64(bk);
            if (lane == 0 && bk) atomicMax(&sh.topkey, bk);
            if (!value_cut<EPT>(sv, s, p.budget, elo, ehi, sh, thr, [&](int j) { return slab_id<NS>(tid, j); })) {
                unsigned long long keys[EPT];
                comm_keys<NS, EPT>(sv, s, keys);
                thr = radix_cut<EPT>(keys, s, false, p.budget, sh);
            }
            if (p.max_comm > 0) {
                unsigned long long keys[EPT];
                comm_keys<NS, EPT>(sv, s, keys);
                thr = umax64(thr, radix_cut<EPT>(keys, s, true, p.max_comm, sh));
            }
            cert = 0u;
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const uint32_t u = ordered_bits(sv[j] == 0.f ? 0.f : sv[j]), c = (uint32_t)slab_id<NS>(tid, j);
                const uint32_t thr_u = (uint32_t)(thr >> 32), thr_id = 0xFFFFFFFFu - (uint32_t)thr;
                if (s[j] > 0 && (u > thr_u || (u == thr_u && c < thr_id))) cert |= 1u << j;
            }
            __syncthreads();
        }
        CKV_TMARK(12);

        // taken communities: the certain ones mark their bits (band members above
        // the band cut are marked already); then every owner reads its bits back
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (any && s[j] > 0 && ((cert >> j) & 1u)) {
                const int c = slab_id<NS>(tid, j);
                atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
            }
        }
        __syncthreads();
        bool taken[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int c = slab_id<NS>(tid, j);
            taken[j] = any && s[j] > 0 && ((sh.bits[c >> 5] >> (c & 31)) & 1u);
        }
        CKV_TMARK(43);
        // Per slab: taken communities and their base members; then taken tail entries.
        constexpr int NV = 2 * NGR + 1;
        static_assert(NV <= 9, "the scan scratch holds nine values per wave");
        int v[NV], ex[NV], tot[NV];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            v[j] = 0;
            v[NGR + j] = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (taken[4 * j + k]) {
                    v[j] += 1;
                    v[NGR + j] += o1(4 * j + k) - o0[4 * j + k];
                }
            }
        }
#pragma unroll
        for (int x = 0; x < X; ++x) {
            const int e = 4 * NS + x;
            v[NS + x] = taken[e] ? 1 : 0;
            v[NGR + NS + x] = taken[e] ? o1(e) - o0[e] : 0;
        }
        int f[kTailPerThread];
        v[2 * NGR] = 0;
#pragma unroll
        for (int j = 0; j < kTailPerThread; ++j) {
            const int i = tid * kTailPerThread + j;
            const int c = tcomm[j];
            f[j] = (i < tn && c >= 0 && c < C && ((sh.bits[c >> 5] >> (c & 31)) & 1u)) ? 1 : 0;
            v[2 * NGR] += f[j];
        }
        block_scan_multi<kSelThreads, NV>(v, ex, tot, sh.scan);
#pragma unroll
        for (int j = 0; j < NGR; ++j) {
            nsel += tot[j];
            ntok += tot[NGR + j];
        }
        ntail = tot[2 * NGR];
        CKV_TMARK(13);

        const int32_t *toks = p.toks + (size_t)g * p.l_cap;
        lds_copy = nsel <= kSelLds;  // uniform
        {
            int kbase = 0, tbase = 0;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                int kpos = kbase + ex[j], rel = tbase + ex[NGR + j];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int e = 4 * j + k;
                    if (taken[e]) {
                        const int len = o1(e) - o0[e];
                        p.sel[(size_t)g * C + kpos] = slab_id<NS>(tid, e);
                        if (lds_copy) {
                            sh.u.cp.soff[kpos] = o0[e];
                            sh.u.cp.spref[kpos] = rel;
                        } else {
                            for (int i = 0; i < len; ++i) tl[ns + rel + i] = toks[o0[e] + i];
                        }
                        rel += len;
                        ++kpos;
                    }
                }
                kbase += tot[j];
                tbase += tot[NGR + j];
            }
#pragma unroll
            for (int x = 0; x < X; ++x) {
                const int e = 4 * NS + x;
                if (taken[e]) {
                    const int kpos = kbase + ex[NS + x], rel = tbase + ex[NGR + NS + x], len = o1(e) - o0[e];
                    p.sel[(size_t)g * C + kpos] = slab_id<NS>(tid, e);
                    if (lds_copy) {
                        sh.u.cp.soff[kpos] = o0[e];
                        sh.u.cp.spref[kpos] = rel;
                    } else {
                        for (int i = 0; i < len; ++i) tl[ns + rel + i] = toks[o0[e] + i];
                    }
                }
                kbase += tot[NS + x];
                tbase += tot[NGR + NS + x];
            }
        }
        for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
        // Taken tail members, in tail order, after the base members.
        {
            int tdst = ns + ntok + ex[2 * NGR];
#pragma unroll
            for (int j = 0; j < kTailPerThread; ++j)
                if (f[j]) tl[tdst++] = tpos[j];
        }
    }
    lds_barrier();  // spref / soff published
    CKV_TMARK(14);
    if (lds_copy) copy_members(p.toks + (size_t)g * p.l_cap, tl, ns, nsel, ntok, sh);
    CKV_TMARK(15);

    if (tid == 0) {
        const unsigned long long tk = sh.topkey;
        p.sel_n[g] = nsel;
        p.tok_n[g] = ns + ntok + ntail;
        p.top[g] = any && tk ? (int)(0xFFFFFFFFu - (uint32_t)tk) : -1;
    }
    CKV_TMARK(16);
}

hipError_t launch_select(const ckv_kv *kv, const ckv_index *idx, const void *q, const float *scores, int budget,
                         int max_comm, int t_cap, int32_t *sel, int32_t *sel_n, int32_t *top,
                         int32_t *tok_list, int32_t *tok_n, const CandArrays &cand, hipStream_t s) {
    SelectParams p{};
    p.cand = cand;
    p.scores = scores;
    p.size = idx->size;
    p.offs = idx->offs;
    p.toks = idx->toks;
    p.tail_pos = idx->tail_pos;
    p.tail_comm = idx->tail_comm;
    p.tail_len = idx->tail_len;
    p.n_comm = idx->n_comm;
    p.seq_len = kv->seq_len;
    p.cscale = idx->cscale;
    p.cent = idx->cent;
    p.q = q;
    p.bf16 = kv->dtype == CKV_DTYPE_BF16;
    p.D = kv->head_dim;
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
    // Whole slabs of 4096, and one column of 1024 more when that covers the
    // rest: 8448 communities take two slabs and a column, not three slabs.
    const int full = idx->c_cap / kSlab, rest = idx->c_cap - full * kSlab;
    const int ns = full >= 1 && rest > 0 && rest <= kSelThreads ? full : ceil_div(idx->c_cap, kSlab);
    const int nx = ns < ceil_div(idx->c_cap, kSlab) ? 1 : 0;
    // candidates per thread: 60 per tile of 256 communities over 1024 threads
    const int nc = ceil_div(cand.ncand, kSelThreads);
    const dim3 grid(w.count), block(kSelThreads);
#define CKV_SEL(N, XX, NN, DD)                                                  \
    if (ns == N && nx == XX && nc == NN && kv->head_dim == DD) {                \
        CKV_LAUNCH((select_kernel<N, XX, NN, DD>), grid, block, s, p);          \
        return hipGetLastError();                                               \
    }
#define CKV_SEL_D(DD)                                                                              \
    CKV_SEL(1, 0, 1, DD) CKV_SEL(1, 1, 1, DD) CKV_SEL(1, 1, 2, DD) CKV_SEL(2, 0, 2, DD)             \
    CKV_SEL(2, 1, 2, DD) CKV_SEL(2, 1, 3, DD) CKV_SEL(3, 0, 3, DD) CKV_SEL(3, 1, 3, DD)             \
    CKV_SEL(3, 1, 4, DD) CKV_SEL(4, 0, 4, DD)
    CKV_SEL_D(64) CKV_SEL_D(128)
#undef CKV_SEL_D
#undef CKV_SEL
    return hipErrorInvalidValue;  // c_cap and head_dim are validated before: not reached
}

// ---------------------------------------------------------------------------
// Centroid budget (the CommunityKV page, Table 6, "Centroid Budget"): the N =
// cent_budget best-ranked non-empty communities that the selection did not
// take, as ascending ids in cent_sel[g][0 .. cent_n[g]).  One 1024-thread
// block per graph; thread t owns communities t, t + 1024, ...  The ranking is
// the selection's (exact score, then lower id), decided from the screening
// intervals [L, U] the same way.  A unit-weight histogram of the outsiders'
// L over 1024 equal-width bins of their score range (a monotone map), walked
// from the top, gives the bin b holding the N-th largest L: N outsiders reach
// a score in bin b or above, so an outsider whose U falls in a lower bin
// cannot be among the N.  The others (typically N and a few) get their exact
// score from the centroid rows and are ranked exactly: each counts the exact
// keys above its own (a radix select for longer lists).  When more than
// kList outsiders reach bin b, every outsider's exact score is computed, slab
// by slab, and a radix select takes the best N.  Fewer than N + 1 outsiders:
// all of them.
constexpr int kCentRankMax = 512;  // candidates ranked by counting; more: radix select

template <int D, int EPT>
__global__ __launch_bounds__(kSelThreads) void centroid_select_kernel(SelectParams p) {
    __shared__ SelShared sh;
    const int g = p.g0 + blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int C = p.c_cap, N = p.cent_budget;
    const int nc = min(p.n_comm[g], C);
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    float sv[EPT], scl[EPT];
    int sz[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid + j * kSelThreads;
        const bool ok = c < nc;
        sv[j] = ok ? p.scores[(size_t)g * C + c] : kNegInf;
        scl[j] = ok ? p.cscale[(size_t)g * C + c] : 0.f;
        sz[j] = ok ? p.size[(size_t)g * C + c] : 0;
    }
    const int ntaken = p.sel_n[g];
    load_qbar(p, gc, sh);
    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;
    sh.bw[tid] = 0;   // kBins == kSelThreads
    sh.bwl[tid] = 0;  // rank counts of the listed candidates
    if (tid == 0) sh.ccount = 0;
    __syncthreads();
    for (int i = tid; i < ntaken; i += kSelThreads) {
        const int c = p.sel[(size_t)g * C + i];
        atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
    }
    float qn = sh.qabs[lane] * (lane < p.D ? 1.f : 0.f);
    if (lane + 64 < p.D) qn += sh.qabs[lane + 64];
    const float kq = wave_sum_f(qn) * kScreenK;
    __syncthreads();

    // Outsiders (non-empty, not taken), their intervals, count and range.
    uint32_t outs = 0u;
    float lw[EPT], up[EPT];
    float blo = -kNegInf, bhi = kNegInf;
    int nout = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid + j * kSelThreads;
        const bool o = sz[j] > 0 && !((sh.bits[c >> 5] >> (c & 31)) & 1u);
        const float e = screen_bound(sv[j], scl[j], kq);
        outs |= (o ? 1u : 0u) << j;
        lw[j] = sv[j] - e;
        up[j] = sv[j] + e;
        if (o) {
            blo = fminf(blo, lw[j]);
            bhi = fmaxf(bhi, up[j]);
            ++nout;
        }
    }
    blo = wave_min_f(blo);
    bhi = wave_max_f(bhi);
    nout = (int)wave_sum_f((float)nout);  // at most 64 * EPT: exact in float32
    if (lane == 0) {
        sh.red_lo[wave] = blo;
        sh.red_hi[wave] = bhi;
        sh.red_lm[wave] = (float)nout;
    }
    __syncthreads();
    nout = 0;
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) {
        blo = fminf(blo, sh.red_lo[i]);
        bhi = fmaxf(bhi, sh.red_hi[i]);
        nout += (int)sh.red_lm[i];
    }
    // From here sh.bits marks the chosen communities.
    for (int i = tid; i < C / 32; i += kSelThreads) sh.bits[i] = 0u;
    __syncthreads();

    if (nout <= N) {  // uniform: every outsider
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int c = tid + j * kSelThreads;
            if ((outs >> j) & 1u) atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
        }
    } else {
        // bin(x) = floor((x - lo) * 1024 / (hi - lo)), clamped: monotone in x.
        const float bscale = bhi > blo ? (float)kBins / (bhi - blo) : 0.f;
        auto bin = [&](float x) { return min(max((int)((x - blo) * bscale), 0), kBins - 1); };
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if ((outs >> j) & 1u) atomicAdd(&sh.bw[bin(lw[j])], 1);
        __syncthreads();
        if (wave == 0) {  // the highest bin b with at least N lower bounds at or above it
            int h[kBins / 64], tot = 0;
#pragma unroll
            for (int i = 0; i < kBins / 64; ++i) {
                h[i] = sh.bw[(kBins / 64) * lane + i];
                tot += h[i];
            }
            int suf = tot;  // this lane and every higher lane
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_down(suf, o, 64);
                if (lane + o < 64) suf += y;
            }
            int acc = suf - tot, found = -1;
#pragma unroll
            for (int i = kBins / 64 - 1; i >= 0; --i) {
                acc += h[i];
                if (found < 0 && acc >= N) found = (kBins / 64) * lane + i;
            }
            const unsigned long long bal = __ballot(found >= 0);
            const int src = bal ? 63 - __clzll((long long)bal) : 0;
            const int fb = __shfl(found, src, 64);
            if (lane == 0) sh.cut_bin = fb;
        }
        __syncthreads();
        const int bcut = sh.cut_bin;  // >= 0: nout > N lower bounds are in the histogram
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (((outs >> j) & 1u) && bin(up[j]) >= bcut) {
                const int slot = atomicAdd(&sh.ccount, 1);
                if (slot < kList) {
                    sh.u.ls.id[slot] = tid + j * kSelThreads;
                    sh.u.ls.sz[slot] = sz[j];
                }
            }
        }
        __syncthreads();
        const int ncand = sh.ccount;
        if (ncand <= kList) {
            exact_scores<D>(p, g, ncand, sh, true, 0);
            __syncthreads();
            constexpr int LPT = kList / kSelThreads;
            unsigned long long k2[LPT];
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const int e = tid + i * kSelThreads;
                k2[i] = e < ncand ? sh.u.ls.key[e] : 0ull;
            }
            unsigned long long t2 = 0ull;  // taken: keys above t2
            if (ncand <= kCentRankMax) {
                // Rank of each key among the candidates' (keys are distinct):
                // candidate e is counted by 1024 / P2 threads (P2 = ncand
                // rounded up to a power of two), each over its own slice of
                // the keys, two keys per 16-byte read; the partial counts
                // meet in sh.bwl.
                const int p2 = ncand <= 1 ? 1 : 1 << (32 - __builtin_clz(ncand - 1));
                const int e = tid & (p2 - 1), parts = kSelThreads / p2;
                const int chunk = ((ncand + parts - 1) / parts + 1) & ~1;
                const int k0 = (tid / p2) * chunk, k1 = min(k0 + chunk, ncand);
                if (e < ncand && k0 < k1) {
                    const unsigned long long mine = sh.u.ls.key[e];
                    int above = 0;
                    for (int k = k0; k < k1; k += 2) {  // k0 even: 16-byte aligned pairs inside key[kList]
                        const ulonglong2 kk = *reinterpret_cast<const ulonglong2 *>(&sh.u.ls.key[k]);
                        above += kk.x > mine ? 1 : 0;
                        above += (k + 1 < k1 && kk.y > mine) ? 1 : 0;
                    }
                    atomicAdd(&sh.bwl[e], above);
                }
                __syncthreads();
                if (tid < ncand && sh.bwl[tid] < N) {
                    const int c = (int)(0xFFFFFFFFu - (uint32_t)k2[0]);
                    atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
                }
            } else {
                int w2[LPT];
#pragma unroll
                for (int i = 0; i < LPT; ++i) w2[i] = 0;
                t2 = radix_cut<LPT>(k2, w2, true, N, sh);
#pragma unroll
                for (int i = 0; i < LPT; ++i) {
                    if (k2[i] && (t2 == 0ull || k2[i] > t2)) {
                        const int c = (int)(0xFFFFFFFFu - (uint32_t)k2[i]);
                        atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
                    }
                }
            }
        } else {  // too many to list: every exact score, slab by slab
            float ex[EPT];
#pragma unroll
            for (int j = 0; j < EPT; ++j) ex[j] = kNegInf;
            for (int sl = 0; sl * kSlab < C; ++sl) {
                const int n = min(kSlab, C - sl * kSlab);
                exact_scores<D>(p, g, n, sh, false, sl);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    const int i = tid + j * kSelThreads - sl * kSlab;
                    if (i >= 0 && i < n) ex[j] = sh.u.exs[i];
                }
                __syncthreads();
            }
            unsigned long long key[EPT];
            int w0[EPT];
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                key[j] = ((outs >> j) & 1u) ? comm_key(ex[j], tid + j * kSelThreads) : 0ull;
                w0[j] = 0;
            }
            const unsigned long long t2 = radix_cut<EPT>(key, w0, true, N, sh);
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                if (key[j] && (t2 == 0ull || key[j] > t2)) {
                    const int c = tid + j * kSelThreads;
                    atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
                }
            }
        }
    }
    __syncthreads();
    // Ascending ids: word w of the bitmap (thread w) writes its communities
    // after those of the words before it.
    const uint32_t word = tid < C / 32 ? sh.bits[tid] : 0u;
    int total;
    int k = block_exclusive_scan<kSelThreads>(__popc(word), sh.scan, &total);
    for (uint32_t m = word; m; m &= m - 1u) p.cent_sel[(size_t)g * N + k++] = tid * 32 + __ffs(m) - 1;
    if (tid == 0) p.cent_n[g] = total;
}

hipError_t launch_centroid_select(const ckv_kv *kv, const ckv_index *idx, const void *q, const float *scores,
                                  const int32_t *sel, const int32_t *sel_n, hipStream_t s) {
    SelectParams p{};
    p.scores = scores;
    p.size = idx->size;
    p.n_comm = idx->n_comm;
    p.cscale = idx->cscale;
    p.cent = idx->cent;
    p.q = q;
    p.bf16 = kv->dtype == CKV_DTYPE_BF16;
    p.D = kv->head_dim;
    p.mode = idx->mode;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.c_cap = idx->c_cap;
    p.sel = const_cast<int32_t *>(sel);
    p.sel_n = const_cast<int32_t *>(sel_n);
    p.cent_budget = idx->cent_budget;
    p.cent_sel = idx->cent_sel;
    p.cent_n = idx->cent_n;
    const Window w = window_of(idx);
    p.g0 = w.first;
    const int ept = ceil_div(idx->c_cap, kSelThreads);
    const dim3 grid(w.count), block(kSelThreads);
#define CKV_CSEL(E, DD)                                                                   \
    if (ept <= E && kv->head_dim == DD) {                                                 \
        hipLaunchKernelGGL((centroid_select_kernel<DD, E>), grid, block, 0, s, p);       \
        return hipGetLastError();                                                         \
    }
#define CKV_CSEL_D(DD) CKV_CSEL(1, DD) CKV_CSEL(2, DD) CKV_CSEL(4, DD) CKV_CSEL(8, DD) CKV_CSEL(12, DD) CKV_CSEL(16, DD)
    CKV_CSEL_D(64) CKV_CSEL_D(128)
#undef CKV_CSEL_D
#undef CKV_CSEL
    return hipErrorInvalidValue;  // c_cap and head_dim are validated before: not reached
}

}  // namespace ckv
