// Split-K combine of one unit's per-block softmax states (the log-sum-exp
// merge of flash decoding): every block that attended a span of the unit's
// tokens leaves, per head, an unnormalised accumulator o[D], its running max m
// and its sum l.  The attention output of the head is
//     M = max_c m_c,  s_c = e^(m_c - M),  L = sum_c l_c s_c,  out = (sum_c o_c s_c) / L.
// Every caller that combines the same records gets the same bits: the gather's
// own last block, and the assign kernel when the gather was launched with its
// combine deferred.  Up to kCombineLds chunks: one wave per head reduces M and
// L over its lanes (lane c holds chunks c, c + 64, ...; L is each lane's fma
// chain over its chunks, then a fixed-order wave sum) and stages s_c in LDS,
// then each (head, dim) sums o_c s_c over the chunks in increasing order as
// one fma chain.  Longer lists (a different, equally fixed order): every
// (head, dim) walks the chunks itself.
#pragma once

#include "ckv_device.h"

namespace ckv {

constexpr int kCombineLds = 256;  // chunks handled by the staged form (four per lane)
constexpr int kCombineLanePass = kCombineLds / 64;
constexpr int kCombineBatch = 32; // accumulator loads in flight per (head, dim) pair and pass

template <int NH>
struct CombineLds {
    float m[NH][kCombineLds];
    float l[NH][kCombineLds];
    float sc[NH][kCombineLds];
    float M[NH];
    float L[NH];
};

// Records of the unit: head h, chunk c at P + (h * nchunk + c) * PS; o in
// [0, D), m at D, l at D + 1.  DEV: written by blocks of the running kernel on
// other XCDs (device-scope loads); otherwise written by an earlier kernel.
template <bool DEV>
__device__ __forceinline__ float ld_part(const float *p) {
    if constexpr (DEV) {
        return ld_dev(p);
    } else {
        return *p;
    }
}

__device__ __forceinline__ float chunk_scale(float m, float M) {
    return (m == kNegInf) ? 0.f : exp2f((m - M) * kLog2e);
}

// Step 1 (nact <= kCombineLds): stage every head's (m, l) into LDS.  The
// caller then synchronises the block (an LDS barrier suffices).
// All loads are issued before the first LDS write (256-thread block).
template <int NH, int D, int PS, bool DEV>
__device__ __forceinline__ void combine_stage(const float *P, int nchunk, int nact, CombineLds<NH> &s) {
    if (nact > kCombineLds) return;
    constexpr int IT = (NH * kCombineLds + 255) / 256;
    float m[IT], l[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int i = threadIdx.x + k * 256;
        const int h = i / nact, c = i - (i / nact) * nact;
        const float *r = P + ((size_t)h * nchunk + c) * PS;
        m[k] = i < NH * nact ? ld_part<DEV>(r + D) : 0.f;
        l[k] = i < NH * nact ? ld_part<DEV>(r + D + 1) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
        const int i = threadIdx.x + k * 256;
        if (i < NH * nact) {
            const int h = i / nact, c = i - (i / nact) * nact;
            s.m[h][c] = m[k];
            s.l[h][c] = l[k];
        }
    }
}

// Step 2 (nact in [1, kCombineLds], all four waves of a 256-thread block):
// wave w reduces the heads w, w + 4, ...: M, the scales s_c and L go to LDS.
// The caller then synchronises the block.
template <int NH>
__device__ __forceinline__ void combine_heads(int nact, CombineLds<NH> &s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int h = wave; h < NH; h += 4) {
        float m[kCombineLanePass];
        float Mlane = kNegInf;
#pragma unroll
        for (int k = 0; k < kCombineLanePass; ++k) {
            const int c = lane + 64 * k;
            m[k] = c < nact ? s.m[h][c] : kNegInf;
            Mlane = fmaxf(Mlane, m[k]);
        }
        const float M = wave_max_f(Mlane);
        float Llane = 0.f;
#pragma unroll
        for (int k = 0; k < kCombineLanePass; ++k) {
            const int c = lane + 64 * k;
            if (c < nact) {
                const float sc = chunk_scale(m[k], M);
                s.sc[h][c] = sc;
                Llane = fmaf(s.l[h][c], sc, Llane);
            }
        }
        const float L = wave_sum_f(Llane);
        if (lane == 0) {
            s.M[h] = M;
            s.L[h] = L;
        }
    }
}

template <int D, int NH, int NT>
constexpr int combine_pairs() {
    return (NH * D + NT - 1) / NT;
}

// nact == 0 (nothing attended): out = 0, ml = (-inf, 0).
template <int D, int NH, int NT>
__device__ __forceinline__ void combine_empty(int t, float *out, float *ml) {
    constexpr int NP = combine_pairs<D, NH, NT>();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = t + i * NT;
        if (pi >= NH * D) continue;
        out[pi] = 0.f;
        if (ml && pi % D == 0) {
            ml[(pi / D) * 2] = kNegInf;
            ml[(pi / D) * 2 + 1] = 0.f;
        }
    }
}

__device__ __forceinline__ void combine_write(int pi, int D, float O, float M, float L, float *out, float *ml) {
    out[pi] = O / L;
    if (ml && pi % D == 0) {
        ml[(pi / D) * 2] = M;
        ml[(pi / D) * 2 + 1] = L;
    }
}

// Step 3 (nact in [1, kCombineLds], after step 2): out[h * D + d] for the
// pairs pi = h * D + d = t, t + NT, ... (t in [0, NT): this thread's index
// among the NT threads that combine); ml[h] = (M, L) when ml is not null.
template <int D, int NH, int PS, bool DEV, int NT>
__device__ __forceinline__ void combine_out(const float *P, int nchunk, int nact, const CombineLds<NH> &s, int t,
                                            float *out, float *ml) {
    constexpr int NP = combine_pairs<D, NH, NT>();
    float O[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) O[i] = 0.f;
    for (int c0 = 0; c0 < nact; c0 += kCombineBatch) {
        float v[NP][kCombineBatch];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pi = t + i * NT;
            const int h = pi / D, d = pi - (pi / D) * D;
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j)
                v[i][j] = (pi < NH * D && c0 + j < nact)
                              ? ld_part<DEV>(P + ((size_t)h * nchunk + c0 + j) * PS + d)
                              : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int pi = t + i * NT;
            if (pi >= NH * D) continue;
            const int h = pi / D;
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j)
                if (c0 + j < nact) O[i] = fmaf(v[i][j], s.sc[h][c0 + j], O[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = t + i * NT;
        if (pi < NH * D) combine_write(pi, D, O[i], s.M[pi / D], s.L[pi / D], out, ml);
    }
}

// Step 3 with the accumulators loaded ahead of time: combine_preload loads
// v[i][j], the entry of pair t + i * NT in chunk j, for every chunk below
// min(lim, NB), possibly before the list length is known (lim = nchunk; the
// records past nact are then loaded but never read).  Requires nact in
// [1, min(NB, lim, kCombineLds)].
template <int D, int NH, int PS, bool DEV, int NT, int NB>
__device__ __forceinline__ void combine_preload(const float *P, int nchunk, int lim, int t,
                                                float (&v)[combine_pairs<D, NH, NT>()][NB]) {
    constexpr int NP = combine_pairs<D, NH, NT>();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = t + i * NT;
        const int h = pi / D, d = pi - (pi / D) * D;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            v[i][j] = (pi < NH * D && j < lim) ? ld_part<DEV>(P + ((size_t)h * nchunk + j) * PS + d) : 0.f;
    }
}

// The same loads with no condition at all: out-of-range pairs and chunks
// read the nearest record entry instead (never used), so every lane and wave
// issues the same loads in the same order.  Records written by an earlier
// kernel; t may be negative (a thread that only loads).
template <int D, int NH, int PS, int NT, int NB>
__device__ __forceinline__ void combine_preload_all(const float *P, int nchunk, int t,
                                                    float (&v)[combine_pairs<D, NH, NT>()][NB]) {
    constexpr int NP = combine_pairs<D, NH, NT>();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = min(max(t + i * NT, 0), NH * D - 1);
        const int h = pi / D, d = pi - (pi / D) * D;
#pragma unroll
        for (int j = 0; j < NB; ++j) v[i][j] = P[((size_t)h * nchunk + min(j, nchunk - 1)) * PS + d];
    }
}

template <int D, int NH, int NT, int NB>
__device__ __forceinline__ void combine_out_regs(int nact, const CombineLds<NH> &s, int t,
                                                 const float (&v)[combine_pairs<D, NH, NT>()][NB], float *out,
                                                 float *ml) {
    constexpr int NP = combine_pairs<D, NH, NT>();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = t + i * NT;
        if (pi >= NH * D) continue;
        const int h = pi / D;
        float O = 0.f;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (j < nact) O = fmaf(v[i][j], s.sc[h][j], O);
        combine_write(pi, D, O, s.M[h], s.L[h], out, ml);
    }
}

// More than kCombineLds chunks: (M, L) of head h read straight from the
// records, L as an fma chain in chunk order.
template <int D, int PS, bool DEV>
__device__ __forceinline__ void head_state_long(const float *P, int nchunk, int nact, int h, float &M, float &L) {
    const float *r = P + (size_t)h * nchunk * PS;
    M = kNegInf;
    for (int c0 = 0; c0 < nact; c0 += kCombineBatch) {
        float mm[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            mm[j] = c0 + j < nact ? ld_part<DEV>(r + (size_t)(c0 + j) * PS + D) : kNegInf;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) M = fmaxf(M, mm[j]);
    }
    L = 0.f;
    for (int c0 = 0; c0 < nact; c0 += kCombineBatch) {
        float mm[kCombineBatch], ll[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            mm[j] = c0 + j < nact ? ld_part<DEV>(r + (size_t)(c0 + j) * PS + D) : kNegInf;
            ll[j] = c0 + j < nact ? ld_part<DEV>(r + (size_t)(c0 + j) * PS + D + 1) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j)
            if (c0 + j < nact) L = fmaf(ll[j], chunk_scale(mm[j], M), L);
    }
}

template <int D, int NH, int PS, bool DEV, int NT>
__device__ __forceinline__ void combine_out_long(const float *P, int nchunk, int nact, int t, float *out, float *ml) {
    constexpr int NP = combine_pairs<D, NH, NT>();
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int pi = t + i * NT;
        if (pi >= NH * D) continue;
        const int h = pi / D, d = pi - (pi / D) * D;
        float M, L;
        head_state_long<D, PS, DEV>(P, nchunk, nact, h, M, L);
        const float *r = P + (size_t)h * nchunk * PS;
        float O = 0.f;
        for (int c0 = 0; c0 < nact; c0 += kCombineBatch) {
            float v[kCombineBatch], mm[kCombineBatch];
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j) {
                v[j] = c0 + j < nact ? ld_part<DEV>(r + (size_t)(c0 + j) * PS + d) : 0.f;
                mm[j] = c0 + j < nact ? ld_part<DEV>(r + (size_t)(c0 + j) * PS + D) : kNegInf;
            }
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j)
                if (c0 + j < nact) O = fmaf(v[j], chunk_scale(mm[j], M), O);
        }
        combine_write(pi, D, O, M, L, out, ml);
    }
}

}  // namespace ckv
