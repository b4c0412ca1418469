// Exact softmax attention over a gathered token list (the CommunityKV page,
// Figure 1 panel (3): exact attention on the retrieved subset together with
// the sink tokens) and the dense flash-decode baseline over every cached token.
//
// One block of 256 threads (4 waves) attends a span of tokens of one unit (a
// graph for the gather, a (sequence, kv head) for the dense baseline).  Each
// token row [K | V] is read by 16 lanes, every lane loading one contiguous
// slice of K and of V (16 B for bf16 d=128), so one wave instruction fetches
// four 256-byte K rows.  All loads of a pass are issued before any arithmetic
// to keep many row fetches in flight.  The q.k dot product is reduced inside
// the 16-lane row with DPP; the softmax state (max, sum, accumulator) is kept
// per lane in float32 and merged across token rows, waves and blocks with the
// usual log-sum-exp rescaling.  The last block of a unit to finish (counted
// with a device-scope atomic that it then resets) merges the per-block
// partials, so the whole split-K attention is one launch.  Blocks of one unit
// run on different XCDs, whose L2 caches are not coherent with each other:
// partial records are padded to whole cache lines and written and read with
// device-scope accesses, and each block waits for its stores before it counts
// itself in.
#include "ckv_device.h"
#include "ckv_internal.h"
#include "combine.h"

namespace ckv {

struct AttendParams {
    const void *kv;
    const int32_t *page_table;
    const int32_t *seq_len;
    int Hq, Hkv, ps_log2, max_pages;
    const void *q;
    const int32_t *tok_list;
    const int32_t *tok_n;
    int t_cap;
    int mode;
    float sm_scale;
    float *out;
    float *logits;
    float *ml;
    float *part;
    int32_t *ctr;
    const int32_t *cent_n;  // gather with a centroid budget: centroid terms per graph (else null)
    int cent_slots;         // record slots of the centroid terms per graph and head
    int nchunk;     // record slots per unit and head
    int dense_tokens;  // dense baseline: tokens per block (a multiple of the pass span)
    int g0;         // first unit of the launch window
    int units;      // units in the launch
};

// The 32-bit words of a row fragment (bf16: two elements each, low half first).
template <int B>
__device__ __forceinline__ void frag_words(const Frag<B> &f, uint32_t (&w)[B / 4]) {
    if constexpr (B == 8) {
        w[0] = f.w.x;
        w[1] = f.w.y;
    } else if constexpr (B == 16) {
        w[0] = f.w.x;
        w[1] = f.w.y;
        w[2] = f.w.z;
        w[3] = f.w.w;
    } else {
        w[0] = f.w0.x;
        w[1] = f.w0.y;
        w[2] = f.w0.z;
        w[3] = f.w0.w;
        w[4] = f.w1.x;
        w[5] = f.w1.y;
        w[6] = f.w1.z;
        w[7] = f.w1.w;
    }
}
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

template <typename T, int D, int NH>
constexpr int pick_u() {
    return (NH >= 8 || RowSlice<T, D>::BYTES == 32) ? 4 : 8;
}

// Combine of the unit's first nrec records into out and ml (the last block of
// the unit, or the first block of a unit whose only records are its centroid
// terms'), then the reset of the unit's arrival counter.
template <int D, int NH, bool DENSE>
__device__ __forceinline__ void attend_combine(const AttendParams &a, int unit, int b, int qh0, int nrec,
                                               CombineLds<NH> &s_comb) {
    constexpr int PS = part_stride(D);
    const int tid = threadIdx.x;
    const float *P = a.part + (size_t)unit * NH * a.nchunk * PS;
    float *o = a.out + ((size_t)b * a.Hq + qh0) * D;
    float *mlu = a.ml ? a.ml + (size_t)unit * NH * 2 : nullptr;
    constexpr int NB = kCombineBatch;
    if (nrec <= NB) {  // accumulators and (m, l) in one round trip
        float v[combine_pairs<D, NH, 256>()][NB];
        combine_preload<D, NH, PS, true, 256, NB>(P, a.nchunk, nrec, tid, v);
        combine_stage<NH, D, PS, true>(P, a.nchunk, nrec, s_comb);
        __syncthreads();
        combine_heads<NH>(nrec, s_comb);
        __syncthreads();
        combine_out_regs<D, NH, 256, NB>(nrec, s_comb, tid, v, o, mlu);
    } else if (nrec <= kCombineLds) {
        combine_stage<NH, D, PS, true>(P, a.nchunk, nrec, s_comb);
        __syncthreads();
        combine_heads<NH>(nrec, s_comb);
        __syncthreads();
        combine_out<D, NH, PS, true, 256>(P, a.nchunk, nrec, s_comb, tid, o, mlu);
    } else {
        combine_out_long<D, NH, PS, true, 256>(P, a.nchunk, nrec, tid, o, mlu);
    }
    if (tid == 0) reset_counter(&a.ctr[unit]);
}

// Block epilogue shared by the gather kernels.  The four waves' softmax states
// (s_wm, s_wl: max and sum per head; s_wacc: unnormalised accumulators) are
// merged in a fixed order into the span's record; a deferred gather stops
// there, a one-span list without centroid terms writes out and ml directly,
// otherwise the last of the unit's nact span blocks combines every span's
// record and the ncent records of the centroid terms after them.
template <int D, int NH, bool DENSE>
__device__ __forceinline__ void attend_finish(const AttendParams &a, int unit, int b, int qh0, int chunk, int nact,
                                              int ncent, bool defer, float (&s_wm)[4][NH], float (&s_wl)[4][NH],
                                              float (&s_wacc)[4][NH][D], CombineLds<NH> &s_comb, int &s_last) {
    constexpr int PS = part_stride(D);
    const int tid = threadIdx.x;
    __syncthreads();

    // Block result per head: merge the four waves in a fixed order.
    float *P = a.part + (size_t)unit * NH * a.nchunk * PS;
    for (int i = tid; i < NH * D; i += 256) {
        const int h = i / D, d = i - (i / D) * D;
        float M = s_wm[0][h];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, s_wm[w][h]);
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float s = (s_wm[w][h] == kNegInf) ? 0.f : exp2f((s_wm[w][h] - M) * kLog2e);
            o += s_wacc[w][h][d] * s;
            L += s_wl[w][h] * s;
        }
        float *dst = P + ((size_t)h * a.nchunk + chunk) * PS;
        if (defer) {  // read by a later kernel: plain stores
            dst[d] = o;
            if (d == 0) {
                dst[D] = M;
                dst[D + 1] = L;
            }
        } else if (nact + ncent == 1) {
            a.out[((size_t)b * a.Hq + qh0 + h) * D + d] = o / L;
            if (a.ml && d == 0) {
                a.ml[((size_t)unit * NH + h) * 2] = M;
                a.ml[((size_t)unit * NH + h) * 2 + 1] = L;
            }
        } else {
            st_dev(dst + d, o);
            if (d == 0) {
                st_dev(dst + D, M);
                st_dev(dst + D + 1, L);
            }
        }
    }
    if constexpr (!DENSE) CKV_TMARK(23);
    if constexpr (!DENSE) CKV_BMARK(3);
    if (nact + ncent == 1 || defer) return;

    // The last block of the unit combines every block's partial.
    stores_done();
    __syncthreads();
    if (tid == 0) s_last = arrive_last(&a.ctr[unit], nact);
    __syncthreads();
    if constexpr (!DENSE) CKV_BMARK(4);
    if (!s_last) return;
    attend_combine<D, NH, DENSE>(a, unit, b, qh0, nact + ncent, s_comb);
    if constexpr (!DENSE) CKV_TMARK(24);
    if constexpr (!DENSE) CKV_BMARK(5);
}

template <typename T, int D, int NH, int U, bool DENSE>
__global__ __launch_bounds__(256) void attend_kernel(AttendParams a) {
    using RS = RowSlice<T, D>;
    constexpr int E = RS::E;
    constexpr int SPAN = 16 * U;
    constexpr int MAX_BLOCK = DENSE ? kDenseTokensMax : kGatherTokens;
    constexpr int ITERS = MAX_BLOCK / SPAN;
    static_assert(MAX_BLOCK % SPAN == 0 && kDenseTokensMin % SPAN == 0, "a block's span is whole passes");
    const int per_block = DENSE ? a.dense_tokens : kGatherTokens;
    constexpr int PS = part_stride(D);
    // Gather with out == nullptr: the combine is deferred to the assign kernel,
    // every block leaves its partial record and the launch ends there.
    const bool defer = !DENSE && a.out == nullptr;

    __shared__ uint32_t s_row[MAX_BLOCK];
    __shared__ float s_q[NH][D];
    __shared__ float s_wm[4][NH], s_wl[4][NH];
    __shared__ float s_wacc[4][NH][D];
    __shared__ CombineLds<NH> s_comb;
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, ts = lane >> 4;
    // Chunk-major order: chunk c of every unit is dispatched before chunk c+1
    // of any, so the short last chunks come last and land where a compute unit
    // already holds two full ones; with a unit count divisible by 8 the blocks
    // of one unit also share an XCD (workgroups go round-robin over the XCDs).
    const int chunk = blockIdx.x / a.units;
    const int lunit = blockIdx.x - chunk * a.units;
    const int unit = a.g0 + lunit;
    if constexpr (!DENSE) CKV_TMARK(20);
    if constexpr (!DENSE) CKV_BMARK(0);

    int b, kh, qh0, n;
    const int start = chunk * per_block;
    // Gather: the span's token positions are loaded together with the list
    // length (start < t_cap always holds, so the loads stay inside the row;
    // entries past the length are ignored), one round trip instead of two.
    constexpr int SLOTS = MAX_BLOCK / 256;
    int pos_l[SLOTS];
    if constexpr (DENSE) {
        b = unit / a.Hkv;
        kh = unit - b * a.Hkv;
        qh0 = kh * NH;
        n = a.seq_len[b];
    } else {
        const GraphCoords gc = graph_coords(unit, a.mode, a.Hq, a.Hkv);
        b = gc.b;
        kh = gc.kh;
        qh0 = gc.qh0;
        const int32_t *tl = a.tok_list + (size_t)unit * a.t_cap + start;
        const int lim = min(per_block, a.t_cap - start);
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int t = tid + i * 256;
            pos_l[i] = t < lim ? tl[t] : 0;
        }
        n = a.tok_n[unit];
    }
    const int ncent = (!DENSE && a.cent_n) ? cent_records(a.cent_n[unit]) : 0;
    if (n <= 0 && chunk == 0 && !defer) {
        if (ncent) {  // centroid terms only: their records are the unit's whole state
            attend_combine<D, NH, DENSE>(a, unit, b, qh0, ncent, s_comb);
            return;
        }
        // nothing to attend: zero output, empty softmax state
        for (int i = tid; i < NH * D; i += 256) a.out[((size_t)b * a.Hq + qh0) * D + i] = 0.f;
        if (a.ml && tid < NH) {
            a.ml[((size_t)unit * NH + tid) * 2] = kNegInf;
            a.ml[((size_t)unit * NH + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    if (start >= n) return;
    const int nact = (n + per_block - 1) / per_block;
    const int cnt = min(per_block, n - start);

    // Stage the row index of every token of the span (rows past the end read
    // position 0 of the sequence, which exists whenever the span is not empty,
    // and are masked below).
    {
        const int32_t *ptab = a.page_table + (size_t)b * a.max_pages;
        const uint32_t smask = (1u << a.ps_log2) - 1u;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int t = tid + i * 256;
            if (t >= per_block) break;
            const int pos = t < cnt ? (DENSE ? start + t : pos_l[i]) : (DENSE ? start : 0);
            const int page = ptab[pos >> a.ps_log2];
            s_row[t] = ((uint32_t)(page * a.Hkv + kh) << a.ps_log2) | ((uint32_t)pos & smask);
        }
        const T *qp = reinterpret_cast<const T *>(a.q) + ((size_t)b * a.Hq + qh0) * D;
        for (int i = tid; i < NH * D; i += 256) s_q[i / D][i % D] = to_f32(qp[i]);
    }
    __syncthreads();

    if constexpr (!DENSE) CKV_TMARK(21);
    if constexpr (!DENSE) CKV_BMARK(1);
    float qr[NH][E];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) qr[h][e] = s_q[h][l16 * E + e];
    // bf16: q.k as packed dot products of element pairs (the products are
    // exact in float32; the pairs' sums round once per pair).  The float32
    // copy of a bf16 q repacks exactly.
    constexpr bool kDot2 = std::is_same<T, bf16_t>::value;
    uint32_t qpk[NH][E / 2];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < E / 2; ++i)
            qpk[h][i] = (__float_as_uint(qr[h][2 * i]) >> 16) | (__float_as_uint(qr[h][2 * i + 1]) & 0xFFFF0000u);

    float m[NH], l[NH], acc[NH][E];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    const T *kvb = reinterpret_cast<const T *>(a.kv);
    for (int it = 0; it < ITERS; ++it) {
        const int base = it * SPAN;
        if (base >= cnt) break;
        typename RS::F kf[U], vf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + u * 16 + wave * 4 + ts;
            const T *row = kvb + (size_t)s_row[t] * (2 * D) + l16 * E;
            kf[u] = RS::load(row);
            vf[u] = RS::load(row + D);
        }
        float z[NH][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + u * 16 + wave * 4 + ts;
            const bool valid = t < cnt;
            float k[E];
            uint32_t kw[RS::BYTES / 4];
            if constexpr (kDot2) frag_words(kf[u], kw);
            else RS::to_float(kf[u], k);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float d = 0.f;
                if constexpr (kDot2) {
#pragma unroll
                    for (int i = 0; i < E / 2; ++i)
                        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, kw[i]),
                                                            __builtin_bit_cast(bf16x2v_t, qpk[h][i]), d, false);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) d = fmaf(qr[h][e], k[e], d);
                }
                d = row16_sum(d);
                z[h][u] = valid ? d * a.sm_scale : kNegInf;
            }
            if constexpr (!DENSE) {
                if (l16 == 0 && valid) {
#pragma unroll
                    for (int h = 0; h < NH; ++h)
                        a.logits[((size_t)unit * NH + h) * a.t_cap + start + t] = z[h][u];
                }
            }
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float mn = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u) mn = fmaxf(mn, z[h][u]);
            const float sc = (m[h] == kNegInf) ? 0.f : exp2f((m[h] - mn) * kLog2e);
            l[h] *= sc;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] *= sc;
            m[h] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[E];
            RS::to_float(vf[u], v);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float p = (z[h][u] == kNegInf) ? 0.f : exp2f((z[h][u] - m[h]) * kLog2e);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
            }
        }
    }

    if constexpr (!DENSE) CKV_TMARK(22);
    if constexpr (!DENSE) CKV_BMARK(2);
    // Merge the four token rows of the wave (lanes l16, l16+16, l16+32, l16+48).
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
            const float mo = shfl_xor_f(m[h], msk), lo = shfl_xor_f(l[h], msk);
            float M, s1, s2;
            softmax_scales(m[h], mo, M, s1, s2);
            l[h] = l[h] * s1 + lo * s2;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float ao = shfl_xor_f(acc[h][e], msk);
                acc[h][e] = acc[h][e] * s1 + ao * s2;
            }
            m[h] = M;
        }
    }
    if (ts == 0) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if (l16 == 0) {
                s_wm[wave][h] = m[h];
                s_wl[wave][h] = l[h];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) s_wacc[wave][h][l16 * E + e] = acc[h][e];
        }
    }
    attend_finish<D, NH, DENSE>(a, unit, b, qh0, chunk, nact, ncent, defer, s_wm, s_wl, s_wacc, s_comb, s_last);
}

// Query groups of four heads (bf16): the q.k products on the matrix cores.
// v_mfma_f32_16x16x32_bf16 takes 16 gathered tokens as the A operand (K rows,
// one 16-byte slice per lane) and the four query heads, padded to 16, as the
// B operand; in the result a lane with l16 = h < 4 holds head h's logits of
// four tokens.  Those 16 lanes apply the softmax with wave-uniform running
// (max, sum) per head and pass the probabilities through LDS to the
// accumulation, which keeps the coalesced layout of the VALU kernel (four
// token rows of 16 lanes, eight dims of V per lane).  With the statistics
// uniform over the wave, its four rows add without rescaling.
typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void attend_group4_kernel(AttendParams a) {
    constexpr int NH = 4;
    constexpr int PER_BLOCK = kGatherTokens;
    constexpr int KS = D / 32;             // k-slices of one 16-token MFMA tile
    constexpr int WT = PER_BLOCK / 4;      // tokens per wave
    constexpr int BT = 32;                 // tokens per batch: two 16-token tiles
    constexpr int E = 8;                   // dims of V per lane
    static_assert(D == 16 * E, "one 16-lane row covers a V row");
    const bool defer = a.out == nullptr;

    __shared__ uint32_t s_row[PER_BLOCK];
    __shared__ float s_wm[4][NH], s_wl[4][NH];
    __shared__ float s_wacc[4][NH][D];
    __shared__ __attribute__((aligned(16))) float s_p[4][BT][NH];
    __shared__ CombineLds<NH> s_comb;
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, ts = lane >> 4;
    const int chunk = blockIdx.x / a.units;
    const int lunit = blockIdx.x - chunk * a.units;
    const int unit = a.g0 + lunit;
    CKV_BMARK(0);
    const GraphCoords gc = graph_coords(unit, a.mode, a.Hq, a.Hkv);
    const int b = gc.b, kh = gc.kh, qh0 = gc.qh0;
    const int start = chunk * PER_BLOCK;
    const int32_t *tl = a.tok_list + (size_t)unit * a.t_cap + start;
    const int pos_l = tid < min(PER_BLOCK, a.t_cap - start) ? tl[tid] : 0;
    const int n = a.tok_n[unit];
    const int ncent = a.cent_n ? cent_records(a.cent_n[unit]) : 0;
    if (n <= 0 && chunk == 0 && !defer) {
        if (ncent) {  // centroid terms only: their records are the unit's whole state
            attend_combine<D, NH, false>(a, unit, b, qh0, ncent, s_comb);
            return;
        }
        // nothing to attend: zero output, empty softmax state
        for (int i = tid; i < NH * D; i += 256) a.out[((size_t)b * a.Hq + qh0) * D + i] = 0.f;
        if (a.ml && tid < NH) {
            a.ml[((size_t)unit * NH + tid) * 2] = kNegInf;
            a.ml[((size_t)unit * NH + tid) * 2 + 1] = 0.f;
        }
        return;
    }
    if (start >= n) return;
    const int nact = (n + PER_BLOCK - 1) / PER_BLOCK;
    const int cnt = min(PER_BLOCK, n - start);
    {
        const int32_t *ptab = a.page_table + (size_t)b * a.max_pages;
        const uint32_t smask = (1u << a.ps_log2) - 1u;
        const int pos = tid < cnt ? pos_l : 0;  // rows past the end read position 0 (masked)
        const int page = ptab[pos >> a.ps_log2];
        s_row[tid] = ((uint32_t)(page * a.Hkv + kh) << a.ps_log2) | ((uint32_t)pos & smask);
    }
    // The heads as the B operand: head l16 (< 4), dims 32 s + 8 ts .. + 8.
    const bf16_t *qp = reinterpret_cast<const bf16_t *>(a.q) + ((size_t)b * a.Hq + qh0 + min(l16, NH - 1)) * D + ts * 8;
    bf16x8v_t qb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8v_t v = *reinterpret_cast<const bf16x8v_t *>(qp + 32 * s);
        qb[s] = l16 < NH ? v : bf16x8v_t{};
    }
    __syncthreads();
    CKV_BMARK(1);

    float m[NH], l[NH], acc[NH][E];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }
    const bf16_t *kvb = reinterpret_cast<const bf16_t *>(a.kv);
    const float c2 = a.sm_scale;
    for (int bt = 0; bt < WT; bt += BT) {
        const int t0 = wave * WT + bt;  // first token of the batch (within the span)
        if (t0 >= cnt) break;           // wave-uniform
        // K slices (A operand: token t0 + 16 g + l16, dims 32 s + 8 ts) and V (row ts of pass p).
        bf16x8v_t ka[2][KS];
        u32x4v_t vf[BT / 4];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const bf16_t *row = kvb + (size_t)s_row[t0 + 16 * g + l16] * (2 * D) + ts * 8;
#pragma unroll
            for (int s = 0; s < KS; ++s)  // streamed once: nontemporal, as RowSlice::load
                ka[g][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8v_t *>(row + 32 * s));
        }
#pragma unroll
        for (int p = 0; p < BT / 4; ++p)
            vf[p] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4v_t *>(kvb + (size_t)s_row[t0 + 4 * p + ts] * (2 * D) + D + l16 * E));
        f32x4v_t sc[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            sc[g] = f32x4v_t{};
#pragma unroll
            for (int s = 0; s < KS; ++s) sc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[g][s], qb[s], sc[g], 0, 0, 0);
        }
        // Lane (ts, l16 = h < 4): head h, tokens t0 + 16 g + 4 ts + i.
        float z[2][4];
        float bmax = kNegInf;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * g + 4 * ts + i;
                z[g][i] = t < cnt ? sc[g][i] * c2 : kNegInf;
                bmax = fmaxf(bmax, z[g][i]);
                if (l16 < NH && t < cnt) a.logits[((size_t)unit * NH + l16) * a.t_cap + start + t] = z[g][i];
            }
        bmax = fmaxf(bmax, shfl_xor_f(bmax, 16));
        bmax = fmaxf(bmax, shfl_xor_f(bmax, 32));
        float mh = kNegInf;  // this lane's head maximum after the update (lanes l16 < 4)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const float mn = fmaxf(m[h], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bmax), h)));
            const float sh = (m[h] == kNegInf) ? 0.f : exp2f((m[h] - mn) * kLog2e);
            l[h] *= sh;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] *= sh;
            m[h] = mn;
            if (l16 == h) mh = mn;
        }
        float psum = 0.f;
        if (l16 < NH) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pr = z[g][i] == kNegInf ? 0.f : exp2f((z[g][i] - mh) * kLog2e);
                    s_p[wave][16 * g + 4 * ts + i][l16] = pr;
                    psum += pr;
                }
        }
        psum += shfl_xor_f(psum, 16);
        psum += shfl_xor_f(psum, 32);
#pragma unroll
        for (int h = 0; h < NH; ++h) l[h] += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(psum), h));
        __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in order: the reads see the writes
#pragma unroll
        for (int p = 0; p < BT / 4; ++p) {
            const float4 pp = *reinterpret_cast<const float4 *>(&s_p[wave][4 * p + ts][0]);
            const uint32_t w4[4] = {vf[p][0], vf[p][1], vf[p][2], vf[p][3]};
            float v[E];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = __uint_as_float(w4[k] << 16);
                v[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
            }
            const float ph[NH] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(ph[h], v[e], acc[h][e]);
        }
        __builtin_amdgcn_wave_barrier();  // the next batch overwrites s_p only after every lane read it
    }
    CKV_BMARK(2);
    // The wave's four token rows share (m, l): their accumulators add.
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            acc[h][e] += shfl_xor_f(acc[h][e], 16);
            acc[h][e] += shfl_xor_f(acc[h][e], 32);
        }
    if (ts == 0) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if (l16 == 0) {
                s_wm[wave][h] = m[h];
                s_wl[wave][h] = l[h];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) s_wacc[wave][h][l16 * E + e] = acc[h][e];
        }
    }
    attend_finish<D, NH, false>(a, unit, b, qh0, chunk, nact, ncent, defer, s_wm, s_wl, s_wacc, s_comb, s_last);
}

template <typename T, int D, int NH, bool DENSE>
static hipError_t launch_t(const AttendParams &p, int units, hipStream_t s) {
    constexpr int U = pick_u<T, D, NH>();
    AttendParams pu = p;
    pu.units = units;
    const int nspan = p.nchunk - p.cent_slots;  // one block per span (the slots after them are the centroids')
    CKV_LAUNCH((attend_kernel<T, D, NH, U, DENSE>), dim3(units * nspan), dim3(256), s, pu);
    return hipGetLastError();
}

template <bool DENSE>
static hipError_t dispatch(const ckv_kv *kv, int nh, const AttendParams &p, int units, hipStream_t s) {
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    const int D = kv->head_dim;
#define CKV_ATT(TT, DD, NN) \
    if (D == DD && nh == NN) return launch_t<TT, DD, NN, DENSE>(p, units, s);
#define CKV_ATT_T(TT)                                                                          \
    CKV_ATT(TT, 64, 1) CKV_ATT(TT, 64, 2) CKV_ATT(TT, 64, 4) CKV_ATT(TT, 64, 8)                \
    CKV_ATT(TT, 128, 1) CKV_ATT(TT, 128, 2) CKV_ATT(TT, 128, 4) CKV_ATT(TT, 128, 8)
    if (bf) {
        CKV_ATT_T(bf16_t)
    } else {
        CKV_ATT_T(float)
    }
#undef CKV_ATT_T
#undef CKV_ATT
    return hipErrorInvalidValue;
}

hipError_t launch_gather(const ckv_kv *kv, const ckv_index *idx, const void *q,
                         const int32_t *tok_list, const int32_t *tok_n, int t_cap, float sm_scale,
                         float *out, float *logits, float *ml, float *part, int32_t *ctr,
                         hipStream_t s) {
    AttendParams p{};
    p.kv = kv->kv;
    p.page_table = kv->page_table;
    p.seq_len = kv->seq_len;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    p.max_pages = kv->max_pages;
    p.q = q;
    p.tok_list = tok_list;
    p.tok_n = tok_n;
    p.t_cap = t_cap;
    p.mode = idx->mode;
    p.sm_scale = sm_scale;
    p.out = out;
    p.logits = logits;
    p.ml = ml;
    p.part = part;
    p.ctr = ctr;
    p.nchunk = gather_slots(idx, t_cap);
    const Window w = window_of(idx);
    p.g0 = w.first;
    const int nh = heads_per_graph(kv, idx);
    if (idx->cent_budget > 0) {  // the centroid terms' records first (no timing events: they stay armed)
        p.cent_n = idx->cent_n;
        p.cent_slots = cent_records(idx->cent_budget);
        const hipError_t e = launch_centroid_attend(kv, idx, q, tok_n, sm_scale, part, p.nchunk, s);
        if (e != hipSuccess) return e;
    }
    if (nh == 4 && kv->head_dim == 128 && kv->dtype == CKV_DTYPE_BF16) {  // query groups of four: matrix cores
        AttendParams pu = p;
        pu.units = w.count;
        CKV_LAUNCH((attend_group4_kernel<128>), dim3(w.count * (p.nchunk - p.cent_slots)), dim3(256), s, pu);
        return hipGetLastError();
    }
    return dispatch<false>(kv, nh, p, w.count, s);
}

hipError_t launch_dense(const ckv_kv *kv, const void *q, float sm_scale, float *out, float *ml,
                        float *part, int32_t *ctr, hipStream_t s) {
    AttendParams p{};
    p.kv = kv->kv;
    p.page_table = kv->page_table;
    p.seq_len = kv->seq_len;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    p.max_pages = kv->max_pages;
    p.q = q;
    p.t_cap = 0;
    p.mode = CKV_MODE_QUERY_GROUP;
    p.sm_scale = sm_scale;
    p.out = out;
    p.ml = ml;
    p.part = part;
    p.ctr = ctr;
    p.dense_tokens = dense_tokens(kv);
    p.nchunk = ceil_div(ctx_cap(kv), p.dense_tokens);
    return dispatch<true>(kv, group_of(kv), p, kv->batch * kv->n_kv_heads, s);
}

}  // namespace ckv
