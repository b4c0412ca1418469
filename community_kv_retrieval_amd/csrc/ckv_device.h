// Device helpers shared by the libckv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

#include "ckv.h"

namespace ckv {

// Phase tracing for profiling builds (CKV_PHASE_TRACE, single translation
// unit): thread 0 of block 0 of a kernel stamps the 100 MHz real-time counter
// into slot `s` of a device array that ckv_trace_read() copies out.  In normal
// builds the marks compile to nothing.
#ifdef CKV_PHASE_TRACE
__device__ unsigned long long g_phase_trace[64];
#define CKV_TMARK(s)                                                   \
    do {                                                               \
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)    \
            ::ckv::g_phase_trace[(s)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
// Per-block stamps of one kernel (slots 0..6 of block blockIdx.x; slot 7 holds
// the hardware id registers of the wave that stamps).
constexpr int kBlockTraceBlocks = 16384;
__device__ unsigned long long g_block_trace[kBlockTraceBlocks * 8];
#define CKV_BMARK(s)                                                                        \
    do {                                                                                    \
        if (threadIdx.x == 0 && blockIdx.x < ::ckv::kBlockTraceBlocks) {                    \
            ::ckv::g_block_trace[blockIdx.x * 8 + (s)] = __builtin_amdgcn_s_memrealtime();  \
            if ((s) == 0)                                                                   \
                ::ckv::g_block_trace[blockIdx.x * 8 + 7] =                                  \
                    ((unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 20) << 32) | \
                    __builtin_amdgcn_s_getreg((31 << 11) | 4);                              \
        }                                                                                   \
    } while (0)
// Event counter in slot s of the phase array (profiling builds: e.g. how often
// a fast path falls back), bumped once per block.
#define CKV_TCOUNT(s)                                                                 \
    do {                                                                              \
        if (threadIdx.x == 0) atomicAdd(&::ckv::g_phase_trace[(s)], 1ull);            \
    } while (0)
// Per-wave stamps of block 0 (slot s of wave w at index 16 s + w).
#define CKV_WMARK(s)                                                                          \
    do {                                                                                      \
        if (blockIdx.x == 0 && blockIdx.y == 0 && (threadIdx.x & 63) == 0)                    \
            ::ckv::g_block_trace[16 * (s) + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
#else
#define CKV_TCOUNT(s) \
    do {              \
    } while (0)
#define CKV_WMARK(s) \
    do {             \
    } while (0)
#define CKV_TMARK(s) \
    do {             \
    } while (0)
#define CKV_BMARK(s) \
    do {             \
    } while (0)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// ---------------------------------------------------------------------------
// One lane's slice of a K or V row.  A row of head_dim elements is spread over
// 16 lanes; lane l16 holds elements [l16*E, l16*E+E), E = D/16.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int BYTES> struct Frag;
template <> struct Frag<8> { uint2 w; };
template <> struct Frag<16> { uint4 w; };
template <> struct Frag<32> { uint4 w0, w1; };

template <typename T, int D> struct RowSlice {
    static constexpr int E = D / 16;
    static constexpr int BYTES = E * (int)sizeof(T);
    typedef Frag<BYTES> F;

    // K/V rows are streamed once per launch: nontemporal loads (no reuse
    // expected in the caches) read randomly placed rows about 8 % faster after
    // a MALL flush and 13 % faster back to back than plain loads, measured
    // with the gather's grid and row pattern.
    __device__ __forceinline__ static F load(const T *p) {
        F f;
        if constexpr (BYTES == 8) {
            const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
            f.w = make_uint2(v.x, v.y);
        } else if constexpr (BYTES == 16) {
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
            f.w = make_uint4(v.x, v.y, v.z, v.w);
        } else {
            const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
            const u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p) + 1);
            f.w0 = make_uint4(a.x, a.y, a.z, a.w);
            f.w1 = make_uint4(b.x, b.y, b.z, b.w);
        }
        return f;
    }

    __device__ __forceinline__ static void to_float(const F &f, float (&x)[E]) {
        uint32_t w[BYTES / 4];
        if constexpr (BYTES == 8) {
            w[0] = f.w.x; w[1] = f.w.y;
        } else if constexpr (BYTES == 16) {
            w[0] = f.w.x; w[1] = f.w.y; w[2] = f.w.z; w[3] = f.w.w;
        } else {
            w[0] = f.w0.x; w[1] = f.w0.y; w[2] = f.w0.z; w[3] = f.w0.w;
            w[4] = f.w1.x; w[5] = f.w1.y; w[6] = f.w1.z; w[7] = f.w1.w;
        }
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = __uint_as_float(w[e]);
        } else {
#pragma unroll
            for (int e = 0; e < E / 2; ++e) {
                x[2 * e] = __uint_as_float(w[e] << 16);
                x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Cross-lane helpers.  Within a row of 16 lanes the butterfly uses DPP:
// quad_perm swaps neighbours and pairs inside a quad, row_half_mirror pairs the
// two quads of each half-row, row_mirror pairs the two half-rows.  After the
// four steps every lane of the row holds the full row reduction.
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kQuadSwap1>(x);
    x += dpp_f<kQuadSwap2>(x);
    x += dpp_f<kRowHalfMirror>(x);
    x += dpp_f<kRowMirror>(x);
    return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// The same butterfly on a float64 (each 32-bit half moved by DPP): every lane
// of the row ends with the identical row sum.
template <int CTRL> __device__ __forceinline__ double dpp_d(double x) {
    const unsigned long long u = __double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double row16_sum_d(double x) {
    x += dpp_d<kQuadSwap1>(x);
    x += dpp_d<kQuadSwap2>(x);
    x += dpp_d<kRowHalfMirror>(x);
    x += dpp_d<kRowMirror>(x);
    return x;
}



// Wave-wide max of a 64-bit key, in every lane: the DPP butterfly inside each
// row of 16 lanes, then the four row results read out with readlane.  Call with
// all 64 lanes active.
template <int CTRL> __device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, true);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
    return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long umin64(unsigned long long a, unsigned long long b) {
    return a < b ? a : b;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
    return ((unsigned long long)hi << 32) | lo;
}
template <bool MAX>
__device__ __forceinline__ unsigned long long wave_ext_u64(unsigned long long x) {
    auto pick = [](unsigned long long a, unsigned long long b) { return MAX ? umax64(a, b) : umin64(a, b); };
    x = pick(x, dpp_u64<kQuadSwap1>(x));
    x = pick(x, dpp_u64<kQuadSwap2>(x));
    x = pick(x, dpp_u64<kRowHalfMirror>(x));
    x = pick(x, dpp_u64<kRowMirror>(x));
    return pick(pick(readlane_u64(x, 0), readlane_u64(x, 16)), pick(readlane_u64(x, 32), readlane_u64(x, 48)));
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) { return wave_ext_u64<true>(x); }
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long x) { return wave_ext_u64<false>(x); }

// Wave-wide 32-bit reductions with the same DPP butterfly (all lanes active).
template <typename F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, F op) {
    auto dpp = [](uint32_t v, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, decltype(ctrl)::value, 0xF, 0xF, true);
    };
    x = op(x, dpp(x, std::integral_constant<int, kQuadSwap1>{}));
    x = op(x, dpp(x, std::integral_constant<int, kQuadSwap2>{}));
    x = op(x, dpp(x, std::integral_constant<int, kRowHalfMirror>{}));
    x = op(x, dpp(x, std::integral_constant<int, kRowMirror>{}));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_max_f(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_min_f(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_sum_f(float x) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
    return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Wave-wide inclusive prefix sum (lane i gets v_0 + ... + v_i), all lanes
// active: shifts by 1, 2, 4 and 8 lanes inside each row of 16 (lanes shifted in
// from outside the row add 0), then row_bcast:15 adds the last lane of rows 0
// and 2 to rows 1 and 3, and row_bcast:31 adds lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Screening code of one centroid element: round(v / scale) clamped to
// [-127, 127], with scale = max |column| / 127, so that
// |v - scale * code| <= scale * (1/2 + 2^-17); a zero scale (all-zero column)
// gives 0.
constexpr float kScreenMax = 127.f;
__device__ __forceinline__ int8_t screen_code(float v, float scale) {
    if (!(scale > 0.f)) return 0;
    const float r = fminf(kScreenMax, fmaxf(-kScreenMax, rintf(v / scale)));
    return (int8_t)(int)r;
}

// Screening bound factor, in units of cscale * |qbar|_1: 1/2 + 2^-17 for the
// rounding of the int8 codes, (D + 4) * 127 * 2^-24 < 0.001 for the float32
// accumulation of D <= 128 products |q_d| * 127 (four partial sums added in
// order) and for rounding qbar to float32, with slack.  A screening score s~
// then lies within E = cscale * |qbar|_1 * kScreenK + 2^-20 |s~| of the exact
// score (the last term for the float32 roundings of s~, of the exact score and
// of s~ +- E).
constexpr float kScreenK = 0.51f;
__device__ __forceinline__ float screen_bound(float s, float cscale, float kq) {
    return cscale * kq + fabsf(s) * 0x1p-20f;
}

// Element (graph g, dim d, community c) of the int8 screening copy, stored
// tile-major: [graph][c_cap / 256][dim][256], so the 256 communities a scoring
// block reads are one contiguous 256 * D-byte region.
__device__ __forceinline__ size_t cq_offset(int g, int d, int c, int D, int c_cap) {
    return (((size_t)g * (c_cap >> 8) + (c >> 8)) * D + d) * 256 + (c & 255);
}

// Order-preserving map of a float32 onto uint32 (larger float, larger code).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-block hand-off inside one kernel.  Blocks of one kernel run on
// different XCDs whose L2 caches are not coherent with each other.  Data meant
// for another block is written and read with device-scope accesses (sc1), which
// go to the device-coherent level.  Before a block announces its data on a
// counter, it waits until its own stores are acknowledged; that is a release
// for sc1 stores without __threadfence()'s write-back and invalidation of the
// whole L2 (which, issued by every block, serialises on the cache).
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every prior load and store acknowledged
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Block barrier for LDS traffic only: waits for this wave's LDS accesses, not
// for its global loads still in flight (their registers are waited for where
// they are used), so loads issued early keep flowing across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Bump a device-scope counter; true for the block that completes `total`.
__device__ __forceinline__ bool arrive_last(int32_t *ctr, int total) {
    return __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
}
__device__ __forceinline__ void reset_counter(int32_t *ctr) {
    __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge two partial softmax states (max m, sum l, unnormalised accumulator).
__device__ __forceinline__ void softmax_scales(float m1, float m2, float &M, float &s1, float &s2) {
    M = fmaxf(m1, m2);
    s1 = (m1 == kNegInf) ? 0.f : exp2f((m1 - M) * kLog2e);
    s2 = (m2 == kNegInf) ? 0.f : exp2f((m2 - M) * kLog2e);
}

// Block-wide exclusive scan of one int per thread (blockDim.x = NT, NT % 64 == 0).
// `scratch` needs NT/64 + 1 ints of shared memory.  Returns the exclusive prefix;
// *total receives the block sum.  Contains two barriers; callers separate two
// scans sharing `scratch` with a barrier.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    if (wave == 0) {  // scan of the wave totals
        const int t = lane < NW ? scratch[lane] : 0;
        int ti = t;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const int y = __shfl_up(ti, o, 64);
            if (lane >= o) ti += y;
        }
        if (lane < NW) scratch[lane] = ti - t;
        if (lane == NW - 1) scratch[NW] = ti;
    }
    __syncthreads();
    *total = scratch[NW];
    return scratch[wave] + x - v;
}

// Coordinates of graph g: sequence, kv head, first query head, query heads.
struct GraphCoords {
    int b, kh, qh0, nh;
};
__device__ __forceinline__ GraphCoords graph_coords(int g, int mode, int n_q_heads, int n_kv_heads) {
    GraphCoords c;
    const int grp = n_q_heads / n_kv_heads;
    if (mode == CKV_MODE_PER_HEAD) {
        c.b = g / n_q_heads;
        const int qh = g - c.b * n_q_heads;
        c.kh = qh / grp;
        c.qh0 = qh;
        c.nh = 1;
    } else {
        c.b = g / n_kv_heads;
        c.kh = g - c.b * n_kv_heads;
        c.qh0 = c.kh * grp;
        c.nh = grp;
    }
    return c;
}

}  // namespace ckv
