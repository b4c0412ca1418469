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
#include <cstdlib>

#include "ckv_device.h"
#include "ckv_internal.h"

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
    int nchunk;     // blocks per unit
    int per_block;  // tokens per block (gather)
    int g0;         // first unit of the launch window
};

template <typename T, int D, int NH>
constexpr int pick_u() {
    return (NH >= 8 || RowSlice<T, D>::BYTES == 32) ? 4 : 8;
}

// Block-wide reduction of NH values per thread (max or sum) over 256 threads;
// every thread gets the results.  red: [4][NH] shared floats.
template <int NH, bool MAX>
__device__ __forceinline__ void block_reduce_nh(float (&v)[NH], float (*red)[NH]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float y = __shfl_xor(v[h], o, 64);
            v[h] = MAX ? fmaxf(v[h], y) : v[h] + y;
        }
        if (lane == 0) red[wave][h] = v[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        float r = red[0][h];
#pragma unroll
        for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, red[w][h]) : r + red[w][h];
        v[h] = r;
    }
    __syncthreads();
}

// Merge the nact partial records (accumulator[D], max, sum) of every head into
// the final output.  Loads are batched so that many are in flight at once.
// Up to kFastMerge partials: the max and sum of every partial go to LDS while
// each thread's accumulator entries are loaded in passes of kMergePass, all in
// the same round trip for the first pass.
constexpr int kFastMerge = 64;
constexpr int kMergePass = 32;

template <int D, int NH, int PS>
__device__ __forceinline__ void merge_partials(const float *P, int nchunk, int nact, float (*s_scale)[256],
                                               float (*s_red)[NH], float *out, float *ml) {
    const int tid = threadIdx.x;
    constexpr int NP = (NH * D + 255) / 256;  // (head, dim) pairs per thread
    if (nact <= kFastMerge) {
        float(*s_m)[kFastMerge] = reinterpret_cast<float(*)[kFastMerge]>(&s_scale[0][0]);
        float(*s_l)[kFastMerge] = reinterpret_cast<float(*)[kFastMerge]>(&s_scale[0][0] + NH * kFastMerge);
        for (int i = tid; i < NH * nact; i += 256) {
            const int h = i / nact, c = i - (i / nact) * nact;
            s_m[h][c] = ld_dev(P + ((size_t)h * nchunk + c) * PS + D);
            s_l[h][c] = ld_dev(P + ((size_t)h * nchunk + c) * PS + D + 1);
        }
        float o[NP][kMergePass];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pi = tid + i * 256;
            const int h = pi / D, d = pi - (pi / D) * D;
#pragma unroll
            for (int c = 0; c < kMergePass; ++c)
                o[i][c] = (pi < NH * D && c < nact) ? ld_dev(P + ((size_t)h * nchunk + c) * PS + d) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pi = tid + i * 256;
            if (pi >= NH * D) break;
            const int h = pi / D, d = pi - (pi / D) * D;
            float M = kNegInf;
            for (int c = 0; c < nact; ++c) M = fmaxf(M, s_m[h][c]);
            float L = 0.f, O = 0.f;
#pragma unroll
            for (int c = 0; c < kMergePass; ++c) {
                if (c < nact) {
                    const float mc = s_m[h][c];
                    const float sc = (mc == kNegInf) ? 0.f : exp2f((mc - M) * kLog2e);
                    L = fmaf(s_l[h][c], sc, L);
                    O = fmaf(o[i][c], sc, O);
                }
            }
            for (int c0 = kMergePass; c0 < nact; c0 += kMergePass) {
                float v[kMergePass];
#pragma unroll
                for (int c = 0; c < kMergePass; ++c)
                    v[c] = (c0 + c < nact) ? ld_dev(P + ((size_t)h * nchunk + c0 + c) * PS + d) : 0.f;
#pragma unroll
                for (int c = 0; c < kMergePass; ++c) {
                    if (c0 + c < nact) {
                        const float mc = s_m[h][c0 + c];
                        const float sc = (mc == kNegInf) ? 0.f : exp2f((mc - M) * kLog2e);
                        L = fmaf(s_l[h][c0 + c], sc, L);
                        O = fmaf(v[c], sc, O);
                    }
                }
            }
            out[pi] = O / L;
            if (ml && d == 0) {
                ml[h * 2] = M;
                ml[h * 2 + 1] = L;
            }
        }
        return;
    }
    float M[NH], L[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) M[h] = kNegInf;
    for (int c = tid; c < nact; c += 256) {
        float m[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) m[h] = ld_dev(P + ((size_t)h * nchunk + c) * PS + D);
#pragma unroll
        for (int h = 0; h < NH; ++h) M[h] = fmaxf(M[h], m[h]);
    }
    block_reduce_nh<NH, true>(M, s_red);

    float o[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) o[i] = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) L[h] = 0.f;
    constexpr int B = 16;
    for (int c0 = 0; c0 < nact; c0 += 256) {
        const int tn = min(256, nact - c0);
        if (tid < tn) {
            float m[NH], l[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                m[h] = ld_dev(P + ((size_t)h * nchunk + c0 + tid) * PS + D);
                l[h] = ld_dev(P + ((size_t)h * nchunk + c0 + tid) * PS + D + 1);
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float sc = (m[h] == kNegInf) ? 0.f : exp2f((m[h] - M[h]) * kLog2e);
                s_scale[h][tid] = sc;
                L[h] += l[h] * sc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pi = tid + i * 256;
            if (pi < NH * D) {
                const int h = pi / D, d = pi - (pi / D) * D;
                const float *src = P + ((size_t)h * nchunk + c0) * PS + d;
                for (int j0 = 0; j0 < tn; j0 += B) {
                    float v[B];
#pragma unroll
                    for (int j = 0; j < B; ++j) v[j] = (j0 + j < tn) ? ld_dev(src + (size_t)(j0 + j) * PS) : 0.f;
#pragma unroll
                    for (int j = 0; j < B; ++j)
                        if (j0 + j < tn) o[i] = fmaf(v[j], s_scale[h][j0 + j], o[i]);
                }
            }
        }
        __syncthreads();
    }
    block_reduce_nh<NH, false>(L, s_red);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = tid + i * 256;
        if (pi < NH * D) {
            const int h = pi / D;
            float Lh = L[0];
#pragma unroll
            for (int hh = 1; hh < NH; ++hh)
                if (h == hh) Lh = L[hh];
            out[pi] = o[i] / Lh;
        }
    }
    if (ml) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
            if (tid == h) {
                ml[h * 2] = M[h];
                ml[h * 2 + 1] = L[h];
            }
    }
}

template <typename T, int D, int NH, int U, bool DENSE>
__global__ __launch_bounds__(256) void attend_kernel(AttendParams a) {
    using RS = RowSlice<T, D>;
    constexpr int E = RS::E;
    constexpr int SPAN = 16 * U;
    constexpr int MAX_BLOCK = DENSE ? kDenseTokens : kGatherMaxTokens;
    const int PER_BLOCK = DENSE ? kDenseTokens : a.per_block;  // a multiple of SPAN, <= MAX_BLOCK
    const int ITERS = PER_BLOCK / SPAN;
    constexpr int PS = part_stride(D);

    __shared__ uint32_t s_row[MAX_BLOCK];
    __shared__ float s_q[NH][D];
    __shared__ float s_wm[4][NH], s_wl[4][NH];
    __shared__ float s_wacc[4][NH][D];
    __shared__ float s_scale[NH][256];
    __shared__ float s_red[4][NH];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, ts = lane >> 4;
    const int lunit = blockIdx.x / a.nchunk;
    const int chunk = blockIdx.x - lunit * a.nchunk;
    const int unit = a.g0 + lunit;
    if constexpr (!DENSE) CKV_TMARK(20);
    if constexpr (!DENSE) CKV_BMARK(0);

    int b, kh, qh0, n;
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
        n = a.tok_n[unit];
    }
    const int start = chunk * PER_BLOCK;
    if (n <= 0 && chunk == 0) {  // nothing to attend: zero output, empty softmax state
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

    // Stage the row index of every token of the span (rows past the end
    // repeat the span's first token and are masked below).
    {
        const int32_t *ptab = a.page_table + (size_t)b * a.max_pages;
        const int32_t *tl = DENSE ? nullptr : a.tok_list + (size_t)unit * a.t_cap + start;
        const uint32_t smask = (1u << a.ps_log2) - 1u;
        for (int t = tid; t < PER_BLOCK; t += 256) {
            const int tt = t < cnt ? t : 0;
            const int pos = DENSE ? start + tt : tl[tt];
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
            float k[E];
            RS::to_float(kf[u], k);
            const int t = base + u * 16 + wave * 4 + ts;
            const bool valid = t < cnt;
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d = fmaf(qr[h][e], k[e], d);
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
        if (nact == 1) {
            a.out[((size_t)b * a.Hq + qh0 + h) * D + d] = o / L;
            if (a.ml && d == 0) {
                a.ml[((size_t)unit * NH + h) * 2] = M;
                a.ml[((size_t)unit * NH + h) * 2 + 1] = L;
            }
        } else {
            float *dst = P + ((size_t)h * a.nchunk + chunk) * PS;
            st_dev(dst + d, o);
            if (d == 0) {
                st_dev(dst + D, M);
                st_dev(dst + D + 1, L);
            }
        }
    }
    if constexpr (!DENSE) CKV_TMARK(23);
    if constexpr (!DENSE) CKV_BMARK(3);
    if (nact == 1) return;

    // The last block of the unit merges every block's partial.
    stores_done();
    __syncthreads();
    if (tid == 0) s_last = arrive_last(&a.ctr[unit], nact);
    __syncthreads();
    if constexpr (!DENSE) CKV_BMARK(4);
    if (!s_last) return;
    merge_partials<D, NH, PS>(P, a.nchunk, nact, s_scale, s_red,
                              a.out + ((size_t)b * a.Hq + qh0) * D,
                              a.ml ? a.ml + (size_t)unit * NH * 2 : nullptr);
    if (tid == 0) reset_counter(&a.ctr[unit]);
    if constexpr (!DENSE) CKV_TMARK(24);
    if constexpr (!DENSE) CKV_BMARK(5);
}

template <typename T, int D, int NH, bool DENSE>
static hipError_t launch_t(const AttendParams &p, int units, hipStream_t s) {
    constexpr int U = pick_u<T, D, NH>();
    CKV_LAUNCH((attend_kernel<T, D, NH, U, DENSE>), dim3(units * p.nchunk), dim3(256), s, p);
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

// Tokens per gather block.  256 (two passes of 128) measured best for every
// workload here: longer spans (512, 1024) pay less per-block staging and
// split-K but lose more to blocks that share a compute unit.
// CKV_GATHER_TOKENS = 512 or 1024 overrides it (tuning).
static int gather_span() {
    if (const char *e = getenv("CKV_GATHER_TOKENS")) {
        const int v = atoi(e);
        if (v == 2 * kGatherTokens || v == kGatherMaxTokens) return v;
    }
    return kGatherTokens;
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
    p.per_block = gather_span();
    p.nchunk = ceil_div(t_cap, p.per_block);
    const Window w = window_of(idx);
    p.g0 = w.first;
    return dispatch<false>(kv, heads_per_graph(kv, idx), p, w.count, s);
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
    p.nchunk = ceil_div(ctx_cap(kv), kDenseTokens);
    return dispatch<true>(kv, group_of(kv), p, kv->batch * kv->n_kv_heads, s);
}

}  // namespace ckv
