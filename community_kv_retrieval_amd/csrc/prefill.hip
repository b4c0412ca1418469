// Prefill graph construction (the CommunityKV page, Figure 1 panel (1)):
// every prompt token becomes a node linked to the kappa earlier tokens it
// attends to most, sink tokens left out of the pool (Table 6); Table 10 times
// this as the prefill's fused top-kappa selection.
//
// The attention logits are a dense contraction, so they run on the matrix
// cores: one wave holds 32 queries of one head as the B operand of
// v_mfma_f32_32x32x16_bf16 and multiplies 32-key tiles of K (the A operand,
// read from LDS) into a 32x32 fp32 tile.  In that tile a lane owns one query
// column and 16 keys, so everything per query stays in the lane: the scores
// are folded into an online log-sum-exp (base 2, the scale entering the
// exponent) and offered to a sorted top-kappa list held in registers; the two
// lanes that share a query merge their states at the end.  Masks are only
// evaluated on the tiles that touch the diagonal, the sinks or the end of
// the prompt.  Four waves of a block use the
// same keys (the heads of one kv head, or four query tiles in group mode), so
// a 64-key tile is staged once per block in LDS, double-buffered, while the
// next one loads.  Tiles are walked in increasing key order and a lane's keys
// in increasing position, so a strict comparison keeps the lower position on
// equal scores.
//
// Graph weights.  One head: the causal softmax probability of the head (the
// list ranks the raw dot products, which order the keys as the logits do for a
// positive scale; the weight is 2^(c s - lse) at the end).  Query group: the sum of the group's head
// probabilities, which needs every head's normaliser first, so a first pass
// writes the per-head log-sum-exp and a second ranks the summed weights.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum PrefillVariant { kPfTopk = 0, kPfTopkW = 1, kPfLse = 2, kPfGroup = 3 };

constexpr int kPfKeys = 64;  // keys per staged tile (two 32-key MFMA tiles)
constexpr int kPfRowPad = 16;  // bytes of padding per staged row (conflict-free 16-byte reads)

struct PrefillParams {
    const uint8_t *kv;       // paged pool
    const int32_t *ptab;     // page table row of the sequence
    const bf16_t *q;         // [n][Hq][D]
    int Hq, Hkv, G, ps_log2;
    int n, n_sinks, kappa;
    float c;                 // sm_scale * log2(e)
    int32_t *edges;          // [graphs][n][kappa]
    float *weights;          // [graphs][n][kappa] or null
    float *lse;              // [Hq][n], log2 domain (group mode)
    int HW;                  // heads per block (per-head variants)
    int nsets;               // head sets (per-head) or kv heads (group)
    int ntg;                 // query-tile groups
};

// Entry (s, p) ranks above (t, r): larger score, then lower position.
__device__ __forceinline__ bool pf_better(float s, int p, float t, int r) {
    return s > t || (s == t && p < r);
}

template <int KL>
__device__ __forceinline__ void pf_insert(float (&ls)[KL], int (&lp)[KL], float s, int p) {
#pragma unroll
    for (int i = KL - 1; i > 0; --i) {
        const bool up = pf_better(s, p, ls[i - 1], lp[i - 1]);
        const bool here = pf_better(s, p, ls[i], lp[i]);
        ls[i] = up ? ls[i - 1] : (here ? s : ls[i]);
        lp[i] = up ? lp[i - 1] : (here ? p : lp[i]);
    }
    if (pf_better(s, p, ls[0], lp[0])) {
        ls[0] = s;
        lp[0] = p;
    }
}

// Insertion of a key visited after every key in the list (a higher
// position): it ranks above an entry only with a strictly larger score.
template <int KL>
__device__ __forceinline__ void pf_insert_later(float (&ls)[KL], int (&lp)[KL], float s, int p) {
#pragma unroll
    for (int i = KL - 1; i > 0; --i) {
        const bool up = s > ls[i - 1];
        const bool here = s > ls[i];
        ls[i] = up ? ls[i - 1] : (here ? s : ls[i]);
        lp[i] = up ? lp[i - 1] : (here ? p : lp[i]);
    }
    if (s > ls[0]) {
        ls[0] = s;
        lp[0] = p;
    }
}

// Key row m of the 32x32 accumulator entry j of lane half `hf`.
__device__ __forceinline__ int pf_row(int j, int hf) { return (j >> 2) * 8 + hf * 4 + (j & 3); }

// Page of every row this thread stages for key tile kt (rows past n repeat the last).
template <int CPR, int NCH>
__device__ __forceinline__ void pf_pages(const PrefillParams &a, int kt, int (&pg)[NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int pos = min(kt * kPfKeys + ((int)threadIdx.x + 256 * i) / CPR, a.n - 1);
        pg[i] = a.ptab[pos >> a.ps_log2];
    }
}

// This thread's 16-byte chunks of the K rows of key tile kt.
template <int D, int CPR, int NCH>
__device__ __forceinline__ void pf_rows(const PrefillParams &a, int kh, int kt, const int (&pg)[NCH],
                                        u32x4_t (&v)[NCH]) {
    const size_t row_bytes = (size_t)D * 2 * 2;  // K row then V row
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = (int)threadIdx.x + 256 * i;
        const int pos = min(kt * kPfKeys + c / CPR, a.n - 1);
        const size_t row = (((size_t)pg[i] * a.Hkv + kh) << a.ps_log2) | (size_t)(pos & ((1 << a.ps_log2) - 1));
        v[i] = *reinterpret_cast<const u32x4_t *>(a.kv + row * row_bytes + (c % CPR) * 16);
    }
}

// 32x32 score tile: the K rows at `arow` (A operand, LDS) times the queries.
template <int KK>
__device__ __forceinline__ f32x16_t pf_mfma(const uint8_t *arow, const bf16x8_t (&qb)[KK]) {
    f32x16_t acc = {};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t *>(arow + kk * 32), qb[kk], acc,
                                                      0, 0, 0);
    return acc;
}

// 2^x as the bare hardware instruction.  A result below the smallest normal
// float comes out as zero, an error under 2^-126 on a softmax term of at most
// 1; exp2f wraps a range test and a rescale around the same instruction, five
// more vector operations per score in the loops below.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// One lane's 16 scores (keys k0 + pf_row(j, hf)) into its log-sum-exp and its
// top-kappa list.  Per head the scores are the raw dot products (the scale is
// positive, so they rank the keys as the logits do; the running maximum m2 is
// kept in the same units and c = sm_scale log2 e enters the exponent as one
// fma); in group mode they are the summed weights.  MASK: the tile touches the
// diagonal, the sinks or the end of the prompt (wave-uniform).
template <int KL, bool LSE, bool TOPK, bool MASK>
__device__ __forceinline__ void pf_scores_m(const PrefillParams &a, const float (&s)[16], int k0, int qp, int hf,
                                            float none, float (&ls)[KL], int (&lp)[KL], float &m2, float &l2) {
    bool att[16], cand[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int kp = k0 + pf_row(j, hf);
        att[j] = !MASK || (kp <= qp && kp < a.n);
        cand[j] = !MASK || (kp >= a.n_sinks && kp < qp && qp < a.n);
    }
    float tmax = kNegInf, cmax = none;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if constexpr (LSE) tmax = fmaxf(tmax, att[j] ? s[j] : kNegInf);
        if constexpr (TOPK) cmax = fmaxf(cmax, cand[j] ? s[j] : none);
    }
    if constexpr (LSE) {
        if (tmax > m2) {
            l2 = m2 == kNegInf ? 0.f : l2 * exp2f((m2 - tmax) * a.c);
            m2 = tmax;
        }
        const float mc = -m2 * a.c;
#pragma unroll
        for (int j = 0; j < 16; ++j) l2 += att[j] ? exp2_hw(fmaf(s[j], a.c, mc)) : 0.f;
    }
    if constexpr (TOPK) {
        if (__builtin_amdgcn_ballot_w64(cmax > ls[KL - 1])) {
            // Each lane pops its own keys above its list minimum, lowest first
            // (later keys come later), one per pass: the wave runs as many
            // passes as its busiest lane has hits.
            uint32_t hits = 0;
            const float thr = ls[KL - 1];
#pragma unroll
            for (int j = 0; j < 16; ++j) hits |= (cand[j] && s[j] > thr) ? (1u << j) : 0u;
            while (__builtin_amdgcn_ballot_w64(hits != 0)) {
                if (hits) {
                    const uint32_t j = (uint32_t)__builtin_ctz(hits);
                    hits &= hits - 1;
                    // s[j] by a tree of bit-masked blends (no indexed access)
                    uint32_t t8[8], t4[4];
                    const uint32_t m0 = 0u - (j & 1u), m1 = 0u - ((j >> 1) & 1u);
                    const uint32_t m2 = 0u - ((j >> 2) & 1u), m3 = 0u - ((j >> 3) & 1u);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t a0 = __float_as_uint(s[2 * i]), a1 = __float_as_uint(s[2 * i + 1]);
                        t8[i] = a0 ^ ((a0 ^ a1) & m0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) t4[i] = t8[2 * i] ^ ((t8[2 * i] ^ t8[2 * i + 1]) & m1);
                    const uint32_t t2a = t4[0] ^ ((t4[0] ^ t4[1]) & m2), t2b = t4[2] ^ ((t4[2] ^ t4[3]) & m2);
                    const float sj = __uint_as_float(t2a ^ ((t2a ^ t2b) & m3));
                    if (sj > ls[KL - 1]) pf_insert_later<KL>(ls, lp, sj, k0 + pf_row((int)j, hf));
                }
            }
        }
    }
}

template <int KL, bool LSE, bool TOPK>
__device__ __forceinline__ void pf_scores(const PrefillParams &a, const float (&s)[16], int k0, int q0, int qp, int hf,
                                          float none, float (&ls)[KL], int (&lp)[KL], float &m2, float &l2) {
    if (k0 + 31 >= q0 || k0 < a.n_sinks || k0 + 31 >= a.n)
        pf_scores_m<KL, LSE, TOPK, true>(a, s, k0, qp, hf, none, ls, lp, m2, l2);
    else
        pf_scores_m<KL, LSE, TOPK, false>(a, s, k0, qp, hf, none, ls, lp, m2, l2);
}

template <int D, int KL, int VAR, int GH>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams a) {
    constexpr int KK = D / 16;           // MFMAs per 32x32 tile
    constexpr int ROWB = D * 2 + kPfRowPad;  // staged row bytes
    constexpr int CPR = D * 2 / 16;      // 16-byte chunks per K row
    constexpr int NCH = kPfKeys * CPR / 256;  // chunks per thread per tile
    constexpr bool kGroup = VAR == kPfGroup;
    constexpr bool kTopk = VAR != kPfLse;
    constexpr bool kLse = VAR == kPfTopkW || VAR == kPfLse;
    constexpr int NQH = kGroup ? GH : 1;  // heads per wave
    const float kNone = kGroup ? -1.f : kNegInf;  // list sentinel (group weights are >= 0)

    __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kPfKeys * ROWB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, qc = lane & 31;
    // Block -> (query-tile group, head set); the latest (longest) tiles first.
    const int tg = a.ntg - 1 - (int)blockIdx.x / a.nsets;
    const int set = (int)blockIdx.x - ((int)blockIdx.x / a.nsets) * a.nsets;
    int kh, head0, tile;
    if constexpr (kGroup) {
        kh = set;
        head0 = kh * a.G;
        tile = tg * 4 + wave;
    } else {
        const int tpb = 4 / a.HW;
        head0 = set * a.HW + (wave % a.HW);
        kh = head0 / a.G;
        tile = tg * tpb + wave / a.HW;
    }
    const int q0 = tile * 32;
    const int qp = q0 + qc;                   // this lane's query position
    const int qlast = q0 < a.n ? min(q0 + 31, a.n - 1) : -1;  // last query of the wave (-1: none)
    // Keys the block needs: up to its last query.
    const int blast = kGroup ? min(tg * 4 * 32 + 127, a.n - 1)
                             : min((tg * (4 / a.HW) + 4 / a.HW) * 32 - 1, a.n - 1);
    const int nkt = blast / kPfKeys + 1;

    // Queries as B operands: query qc, dims kk*16 + hf*8 .. +8 (clamped rows past n are never used).
    bf16x8_t qb[NQH][KK];
#pragma unroll
    for (int h = 0; h < NQH; ++h) {
        const bf16_t *qr = a.q + ((size_t)min(qp, a.n - 1) * a.Hq + head0 + h) * D + hf * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qb[h][kk] = *reinterpret_cast<const bf16x8_t *>(qr + kk * 16);
    }
    float lse_q[NQH];  // group: the heads' log2 normalisers of this lane's query
    if constexpr (kGroup) {
#pragma unroll
        for (int h = 0; h < NQH; ++h) lse_q[h] = a.lse[(size_t)(head0 + h) * a.n + min(qp, a.n - 1)];
    }

    float ls[KL];
    int lp[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) {
        ls[i] = kNone;
        lp[i] = 0x7FFFFFFF;
    }
    float m2 = kNegInf, l2 = 0.f;  // online log-sum-exp state (log2 domain)

    // Staging: thread t moves chunks t + 256 i (row c / CPR, column c % CPR).
    // Two register sets alternate, so the rows of tile kt + 2 are in flight
    // while tile kt is computed (and the page-table entries two tiles further).
    int pgA[NCH], pgB[NCH];
    u32x4_t stA[NCH], stB[NCH];
    pf_pages<CPR, NCH>(a, 0, pgA);
    pf_rows<D, CPR, NCH>(a, kh, 0, pgA, stA);
    if (nkt > 2) pf_pages<CPR, NCH>(a, 2, pgA);
    if (nkt > 1) {
        pf_pages<CPR, NCH>(a, 1, pgB);
        pf_rows<D, CPR, NCH>(a, kh, 1, pgB, stB);
        if (nkt > 3) pf_pages<CPR, NCH>(a, 3, pgB);
    }

    auto key_tile = [&](int kt, u32x4_t (&stg)[NCH], int (&pg)[NCH]) __attribute__((always_inline)) {
        uint8_t *buf = s_k[kt & 1];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u32x4_t *>(buf + (c / CPR) * ROWB + (c % CPR) * 16) = stg[i];
        }
        __syncthreads();
        if (kt + 2 < nkt) {
            pf_rows<D, CPR, NCH>(a, kh, kt + 2, pg, stg);
            if (kt + 4 < nkt) pf_pages<CPR, NCH>(a, kt + 4, pg);
        }
        const int k0 = kt * kPfKeys;
        if (k0 > qlast) return;  // wave-uniform: past this wave's queries
        const bool two = k0 + 32 <= qlast;
        const uint8_t *r0 = buf + qc * ROWB + hf * 16;
        const uint8_t *r1 = r0 + 32 * ROWB;
        // Scores of this lane's query against keys k0 + [0, 32) and k0 + [32, 64)
        // (entry j: key pf_row(j, hf)), log2 domain; both MFMA chains are issued
        // before the scores of the first are used.
        float s0[16], s1[16];
        if constexpr (kGroup) {
#pragma unroll
            for (int j = 0; j < 16; ++j) s0[j] = s1[j] = 0.f;
#pragma unroll
            for (int h = 0; h < NQH; ++h) {
                const f32x16_t acc0 = pf_mfma<KK>(r0, qb[h]);
                f32x16_t acc1 = {};
                if (two) acc1 = pf_mfma<KK>(r1, qb[h]);
#pragma unroll
                for (int j = 0; j < 16; ++j) s0[j] += exp2_hw(fmaf(acc0[j], a.c, -lse_q[h]));
                if (two) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) s1[j] += exp2_hw(fmaf(acc1[j], a.c, -lse_q[h]));
                }
            }
        } else {
            const f32x16_t acc0 = pf_mfma<KK>(r0, qb[0]);
            f32x16_t acc1 = {};
            if (two) acc1 = pf_mfma<KK>(r1, qb[0]);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s0[j] = acc0[j];
                s1[j] = acc1[j];
            }
        }
        pf_scores<KL, kLse, kTopk>(a, s0, k0, q0, qp, hf, kNone, ls, lp, m2, l2);
        if (two) pf_scores<KL, kLse, kTopk>(a, s1, k0 + 32, q0, qp, hf, kNone, ls, lp, m2, l2);
    };
    for (int kt = 0; kt < nkt; kt += 2) {
        key_tile(kt, stA, pgA);
        if (kt + 1 < nkt) key_tile(kt + 1, stB, pgB);
    }

    // The two lanes of each query (qc, qc + 32) merge their states.
    if constexpr (kLse) {
        const float mo = __shfl_xor(m2, 32, 64), lo = __shfl_xor(l2, 32, 64);
        const float M = fmaxf(m2, mo);
        const float L = (m2 == kNegInf ? 0.f : l2 * exp2f((m2 - M) * a.c)) +
                        (mo == kNegInf ? 0.f : lo * exp2f((mo - M) * a.c));
        m2 = M * a.c + log2f(L);  // the query's log-sum-exp of the logits, log2 domain
    }
    if constexpr (kTopk) {
        float os[KL];
        int op[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            os[i] = __shfl_xor(ls[i], 32, 64);
            op[i] = __shfl_xor(lp[i], 32, 64);
        }
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (os[i] != kNone && pf_better(os[i], op[i], ls[KL - 1], lp[KL - 1])) pf_insert<KL>(ls, lp, os[i], op[i]);
    }
    if (hf != 0 || qp >= a.n) return;
    if constexpr (VAR == kPfLse) {
        a.lse[(size_t)head0 * a.n + qp] = m2;
    } else {
        const int g = kGroup ? kh : head0;
        int32_t *e = a.edges + ((size_t)g * a.n + qp) * a.kappa;
        float *w = a.weights ? a.weights + ((size_t)g * a.n + qp) * a.kappa : nullptr;
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            if (i >= a.kappa) break;
            const bool has = ls[i] != kNone;
            e[i] = has ? lp[i] : -1;
            if (w) {
                float wt = 0.f;
                if (has) wt = kGroup ? ls[i] : exp2f(fmaf(ls[i], a.c, -m2));
                w[i] = wt;
            }
        }
    }
}

template <int D, int KL, int VAR, int GH>
static hipError_t pf_launch(const PrefillParams &p, int blocks, hipStream_t s) {
    CKV_LAUNCH((prefill_kernel<D, KL, VAR, GH>), dim3(blocks), dim3(256), s, p);
    return hipGetLastError();
}

template <int D, int KL>
static hipError_t pf_dispatch(const PrefillParams &p, int var, int blocks, hipStream_t s) {
    switch (var) {
    case kPfTopk: return pf_launch<D, KL, kPfTopk, 1>(p, blocks, s);
    case kPfTopkW: return pf_launch<D, KL, kPfTopkW, 1>(p, blocks, s);
    case kPfLse: return pf_launch<D, 8, kPfLse, 1>(p, blocks, s);
    default: break;
    }
    if constexpr (KL <= 16) {
        if (p.G == 1) return pf_launch<D, KL, kPfGroup, 1>(p, blocks, s);
        if (p.G == 2) return pf_launch<D, KL, kPfGroup, 2>(p, blocks, s);
        if (p.G == 4) return pf_launch<D, KL, kPfGroup, 4>(p, blocks, s);
    }
    return hipErrorInvalidValue;
}

static hipError_t pf_run(const PrefillParams &p, int D, int kl, int var, int blocks, hipStream_t s) {
    if (D == 128) {
        if (kl == 8) return pf_dispatch<128, 8>(p, var, blocks, s);
        if (kl == 16) return pf_dispatch<128, 16>(p, var, blocks, s);
        return pf_dispatch<128, 32>(p, var, blocks, s);
    }
    if (kl == 8) return pf_dispatch<64, 8>(p, var, blocks, s);
    if (kl == 16) return pf_dispatch<64, 16>(p, var, blocks, s);
    return pf_dispatch<64, 32>(p, var, blocks, s);
}

hipError_t launch_prefill(const ckv_kv *kv, int mode, int b, const void *q, int n, int n_sinks, int kappa,
                          float sm_scale, int32_t *edges, float *weights, float *lse, hipStream_t s) {
    PrefillParams p{};
    p.kv = reinterpret_cast<const uint8_t *>(kv->kv);
    p.ptab = kv->page_table + (size_t)b * kv->max_pages;
    p.q = reinterpret_cast<const bf16_t *>(q);
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.G = kv->n_q_heads / kv->n_kv_heads;
    p.ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    p.n = n;
    p.n_sinks = n_sinks;
    p.kappa = kappa;
    p.c = sm_scale * 1.4426950408889634f;
    p.edges = edges;
    p.weights = weights;
    p.lse = lse;
    const int kl = kappa <= 8 ? 8 : kappa <= 16 ? 16 : 32;
    const int D = kv->head_dim;
    const int ntiles = ceil_div(n, 32);
    if (mode == CKV_MODE_PER_HEAD) {
        p.HW = p.G < 4 ? p.G : 4;
        p.nsets = p.Hq / p.HW;
        p.ntg = ceil_div(ntiles, 4 / p.HW);
        return pf_run(p, D, kl, weights ? kPfTopkW : kPfTopk, p.nsets * p.ntg, s);
    }
    // Query groups: every head's log-sum-exp, then the summed weights.
    p.HW = p.G < 4 ? p.G : 4;
    p.nsets = p.Hq / p.HW;
    p.ntg = ceil_div(ntiles, 4 / p.HW);
    hipError_t e = pf_run(p, D, 8, kPfLse, p.nsets * p.ntg, s);
    if (e != hipSuccess) return e;
    p.nsets = p.Hkv;
    p.ntg = ceil_div(ntiles, 4);
    return pf_run(p, D, kl, kPfGroup, p.nsets * p.ntg, s);
}

}  // namespace ckv
