// Budgeted community retrieval (the CommunityKV page, Figure 1 panel (3):
// retrieve a candidate subset of communities under a token budget).
//
// One 1024-thread block per graph; thread t owns the EPT consecutive
// communities t*EPT ... .  Communities rank by float32 score, higher first,
// ties to the lower id; as one number that is the 64-bit key
// (order-preserving bits of the score) << 32 | (~id).  The taken set is the
// longest prefix of the ranking that fits the budget, i.e. every key above the
// key of the first community that overflows it (the cut).
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
// Then the taken ids are compacted in ascending id order with block scans, and
// the attended token list is written: sinks, the base members of every taken
// community, then the taken communities' tail members.  Sizes, scores, CSR
// offsets and tail entries are read at the start with 16-byte loads.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kBins = kSelThreads;
// Member slots mapped to their community in LDS (the common case); longer
// lists binary-search the communities' first slots (up to kSelLds
// communities), and more communities than that are copied one thread each.
constexpr int kSelSlots = 4096;
constexpr int kSelLds = 2048;
constexpr int kSlotsPerThread = kSelSlots / kSelThreads;
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
    int owner[kSelSlots];    // member slot -> index of its taken community
    int soff[kSelLds];       // first base member in toks of the k-th taken community
    int spref[kSelLds + 1];  // its first slot in the token list (after the sinks)
    int bw[kBins];           // token weight per score bin
    uint32_t hw[256];        // radix select: token weight per digit
    uint32_t hn[256];        // radix select: candidates per digit
    uint32_t bits[CKV_MAX_C_CAP / 32];
    unsigned long long ckey[64];
    int csz[64];
    int ccount;
    int cut_bin, cut_above;
    int scan[kSelThreads / 64 + 1];
    float red_lo[kSelThreads / 64], red_hi[kSelThreads / 64];
    uint32_t red_id[kSelThreads / 64];
    unsigned long long prefix, mask, thr;
    long long rem;
    int done;
};

__device__ __forceinline__ unsigned long long comm_key(float s, int c) {
    return ((unsigned long long)ordered_bits(s) << 32) | (0xFFFFFFFFu - (uint32_t)c);
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
        key[j] = w[j] > 0 ? comm_key(sv[j], tid * EPT + j) : 0ull;
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

// Budget cut through equal-width score bins (see the file comment).  Returns
// false, uniformly across the block, when the radix select has to decide.
template <int EPT>
__device__ bool value_cut(const float (&sv)[EPT], const int (&w)[EPT], int budget, float lo, float hi,
                          SelShared &sh, unsigned long long &thr) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float scale = (float)kBins / (hi - lo);
    if (!(hi > lo) || !(scale < __builtin_huge_valf())) return false;
    sh.bw[tid] = 0;
    if (tid == 0) sh.ccount = 0;
    __syncthreads();
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
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
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
        __syncthreads();
        return true;
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (bin[j] == cb) {
            const int i = atomicAdd(&sh.ccount, 1);
            if (i < 64) {
                sh.ckey[i] = comm_key(sv[j], tid * EPT + j);
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

    // Sizes, scores and CSR offsets of this thread's EPT consecutive
    // communities, 16 bytes per load, and the tail entries.
    static_assert(EPT % 4 == 0, "EPT must be a multiple of 4");
    int s[EPT], o0[EPT], o1[EPT];
    float sv[EPT];
    {
        // c % 4 == 0 and C % 256 == 0: a 16-byte load from c < C stays inside
        // the row (the offsets row holds C + 4 entries).  Nothing waits for
        // n_comm: entries at or past it are masked below.
        int4 s4[EPT / 4], o4[EPT / 4];
        float4 v4[EPT / 4];
        int olast = 0;
#pragma unroll
        for (int j = 0; j < EPT; j += 4) {
            const int c = tid * EPT + j;
            s4[j / 4] = make_int4(0, 0, 0, 0);
            o4[j / 4] = make_int4(0, 0, 0, 0);
            v4[j / 4] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < C) {
                s4[j / 4] = *reinterpret_cast<const int4 *>(sz + c);
                v4[j / 4] = *reinterpret_cast<const float4 *>(sc + c);
                o4[j / 4] = *reinterpret_cast<const int4 *>(offs + c);
            }
        }
        if (tid * EPT + EPT <= C) olast = offs[tid * EPT + EPT];
#pragma unroll
        for (int j = 0; j < EPT; j += 4) {
            const int c = tid * EPT + j;
            s[j] = c < nc ? s4[j / 4].x : 0;
            s[j + 1] = c + 1 < nc ? s4[j / 4].y : 0;
            s[j + 2] = c + 2 < nc ? s4[j / 4].z : 0;
            s[j + 3] = c + 3 < nc ? s4[j / 4].w : 0;
            sv[j] = v4[j / 4].x;
            sv[j + 1] = v4[j / 4].y;
            sv[j + 2] = v4[j / 4].z;
            sv[j + 3] = v4[j / 4].w;
            o0[j] = o4[j / 4].x;
            o0[j + 1] = o4[j / 4].y;
            o0[j + 2] = o4[j / 4].z;
            o0[j + 3] = o4[j / 4].w;
        }
#pragma unroll
        for (int j = 0; j + 1 < EPT; ++j) o1[j] = o0[j + 1];
        o1[EPT - 1] = olast;
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
    // Best-ranked community: the lowest id among those scoring hi.
    uint32_t best = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
        if (s[j] > 0 && sv[j] == hi) best = min(best, (uint32_t)(tid * EPT + j));
    best = wave_min_u32(best);
    if (lane == 0) sh.red_id[wave] = best;
    __syncthreads();
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
    int nloc = 0, tokloc = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const uint32_t u = ordered_bits(sv[j]), c = (uint32_t)(tid * EPT + j);
        taken[j] = s[j] > 0 && (u > thr_u || (u == thr_u && c < thr_id));
        if (taken[j]) {
            ++nloc;
            tokloc += o1[j] - o0[j];
        }
    }
    int nsel, ntok;
    int kpos = block_exclusive_scan<kSelThreads>(nloc, sh.scan, &nsel);
    __syncthreads();
    int dst = ns + block_exclusive_scan<kSelThreads>(tokloc, sh.scan, &ntok);
    __syncthreads();
    CKV_TMARK(13);
    const int32_t *toks = p.toks + (size_t)g * p.l_cap;
    const int mode = nsel > kSelLds ? 2 : (ntok <= kSelSlots ? 0 : 1);  // uniform
    if (mode == 0)
        for (int j = tid; j < ntok; j += kSelThreads) sh.owner[j] = -1;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (taken[j]) {
            const int c = tid * EPT + j;
            const int rel = dst - ns, len = o1[j] - o0[j];
            p.sel[(size_t)g * C + kpos] = c;
            atomicOr(&sh.bits[c >> 5], 1u << (c & 31));
            if (mode < 2) {
                sh.soff[kpos] = o0[j];
                sh.spref[kpos] = rel;
                if (mode == 0 && len > 0) sh.owner[rel] = kpos;  // first slot of the community
            } else {
                for (int i = 0; i < len; ++i) tl[dst + i] = toks[o0[j] + i];
            }
            dst += len;
            ++kpos;
        }
    }
    if (tid == 0 && mode == 1) sh.spref[nsel] = ntok;
    for (int i = tid; i < ns; i += kSelThreads) tl[i] = i;
    __syncthreads();
    CKV_TMARK(14);
    if (mode == 0) {
        // every slot takes the owner of the nearest marked slot at or before it:
        // an inclusive prefix max over kSlotsPerThread consecutive slots per thread
        int ow[kSlotsPerThread], run = -1;
#pragma unroll
        for (int u = 0; u < kSlotsPerThread; ++u) {
            const int j = tid * kSlotsPerThread + u;
            ow[u] = j < ntok ? sh.owner[j] : -1;
            run = max(run, ow[u]);
            ow[u] = run;
        }
        const int before = block_inclusive_max<kSelThreads>(run, sh.scan);
        const int carry = __shfl_up(before, 1, 64);
        int prev = (tid & 63) ? carry : -1;
        if ((tid & 63) == 0 && tid > 0) prev = sh.scan[(tid >> 6)];  // max over earlier waves
        int v[kSlotsPerThread];
#pragma unroll
        for (int u = 0; u < kSlotsPerThread; ++u) {
            const int j = tid * kSlotsPerThread + u;
            const int k = max(prev, ow[u]);
            v[u] = j < ntok ? toks[sh.soff[k] + (j - sh.spref[k])] : 0;
        }
#pragma unroll
        for (int u = 0; u < kSlotsPerThread; ++u) {
            const int j = tid * kSlotsPerThread + u;
            if (j < ntok) tl[ns + j] = v[u];
        }
    } else if (mode == 1) {
        for (int j0 = 0; j0 < ntok; j0 += 4 * kSelThreads) {
            int v[4], at[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * kSelThreads + tid;
                at[u] = j;
                if (j < ntok) {  // the last taken community whose first slot is <= j
                    int a = 0, b = nsel - 1;
                    while (a < b) {
                        const int mid = (a + b + 1) >> 1;
                        if (sh.spref[mid] <= j) a = mid;
                        else b = mid - 1;
                    }
                    v[u] = toks[sh.soff[a] + (j - sh.spref[a])];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (at[u] < ntok) tl[ns + at[u]] = v[u];
        }
    }
    CKV_TMARK(15);

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
    const int ept = ceil_div(idx->c_cap, kSelThreads);
    const dim3 grid(idx->n_graphs), block(kSelThreads);
    if (ept <= 4) CKV_LAUNCH((select_kernel<4>), grid, block, s, p);
    else if (ept <= 8) CKV_LAUNCH((select_kernel<8>), grid, block, s, p);
    else if (ept <= 12) CKV_LAUNCH((select_kernel<12>), grid, block, s, p);
    else CKV_LAUNCH((select_kernel<16>), grid, block, s, p);
    return hipGetLastError();
}

}  // namespace ckv
