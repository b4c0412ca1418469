// Read ceiling of the gather's access pattern (a measurement aid, no part of
// the method).  It reads given K|V rows of the paged store exactly as the
// gather does, 256 rows per block staged in LDS, 16 lanes per row, the same
// fragments per lane and rows in flight, with no arithmetic beyond an XOR
// checksum of the bytes read.  Its rate is the practical HBM read rate of
// randomly placed rows, reported beside the 8 TB/s peak; the checksum lets a
// test confirm that every byte was read.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

template <int B>
__device__ __forceinline__ uint32_t frag_xor(const Frag<B> &f) {
    if constexpr (B == 8) {
        return f.w.x ^ f.w.y;
    } else if constexpr (B == 16) {
        return f.w.x ^ f.w.y ^ f.w.z ^ f.w.w;
    } else {
        return f.w0.x ^ f.w0.y ^ f.w0.z ^ f.w0.w ^ f.w1.x ^ f.w1.y ^ f.w1.z ^ f.w1.w;
    }
}

template <typename T, int D, int U>
__global__ __launch_bounds__(256) void read_rows_kernel(const T *kv, const uint32_t *rows, int n, uint32_t n_rows,
                                                        uint32_t *part) {
    using RS = RowSlice<T, D>;
    constexpr int PER_BLOCK = kGatherTokens;
    constexpr int SPAN = 16 * U;
    static_assert(PER_BLOCK % SPAN == 0 && PER_BLOCK == 256, "one row per thread, whole passes");
    __shared__ uint32_t s_row[PER_BLOCK];
    __shared__ uint32_t s_x[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, ts = lane >> 4;
    const int start = blockIdx.x * PER_BLOCK;
    const int cnt = min(PER_BLOCK, n - start);  // >= 1: the grid covers n exactly
    // Row ids past the store are clamped to its last row; slots past the end
    // read row 0 and are left out of the checksum.
    s_row[tid] = tid < cnt ? min(rows[start + tid], n_rows - 1u) : 0u;
    __syncthreads();
    uint32_t x = 0u;
    for (int base = 0; base < cnt; base += SPAN) {  // uniform
        typename RS::F kf[U], vf[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const T *row = kv + (size_t)s_row[base + u * 16 + wave * 4 + ts] * (2 * D) + l16 * RS::E;
            kf[u] = RS::load(row);
            vf[u] = RS::load(row + D);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * 16 + wave * 4 + ts < cnt) x ^= frag_xor(kf[u]) ^ frag_xor(vf[u]);
    }
    x = wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a ^ b; });
    if (lane == 0) s_x[wave] = x;
    __syncthreads();
    if (tid == 0) part[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

hipError_t launch_read_rows(const ckv_kv *kv, const uint32_t *rows, int n, uint32_t *part, hipStream_t s) {
    const uint32_t n_rows = (uint32_t)((long long)kv->n_pages * kv->n_kv_heads * kv->page_size);
    const dim3 grid(ceil_div(n, kGatherTokens)), block(256);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
#define CKV_RR(TT, DD)                                                                                   \
    if (kv->head_dim == DD) {                                                                            \
        constexpr int U = RowSlice<TT, DD>::BYTES == 32 ? 4 : 8;                                         \
        CKV_LAUNCH((read_rows_kernel<TT, DD, U>), grid, block, s, reinterpret_cast<const TT *>(kv->kv), rows, n, \
                   n_rows, part);                                                                        \
        return hipGetLastError();                                                                        \
    }
    if (bf) {
        CKV_RR(bf16_t, 64) CKV_RR(bf16_t, 128)
    } else {
        CKV_RR(float, 64) CKV_RR(float, 128)
    }
#undef CKV_RR
    return hipErrorInvalidValue;
}

}  // namespace ckv
