// Centroid scoring (the CommunityKV page, Figure 1 panel (3): score the query
// against the community centroids; Table 1: retrieval is one pass over the
// centroids).
//
// The scores are a matrix-vector product per graph, s = cent^T qbar, streamed
// once from HBM at 0.5 flop/byte, so the kernel is bandwidth-bound and runs on
// the vector units, not the matrix cores.  The centroid table is stored
// transposed, [graph][dim][community], so lane j of a wave owns communities
// 4j..4j+3 of a 256-wide tile and every wave instruction reads 1 KB of one
// dimension's row with 16-byte loads; no cross-lane reduction is needed.  The
// four waves of a block split the dimensions and add their partial sums in a
// fixed order.  Products and sums are float64 (float32 centroid times a bf16 or
// fp32 query is exact in float64), rounded once to float32 at the end.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

struct ScoreParams {
    const void *q;
    const float *cent;
    const int32_t *size;
    const int32_t *n_comm;
    float *scores;
    int mode, Hq, Hkv, c_cap, g0;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
    __shared__ double s_q[D];
    __shared__ double s_part[4][256];
    const int g = p.g0 + blockIdx.y, c0 = blockIdx.x * 256;
    CKV_TMARK(0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nc = min(p.n_comm[g], p.c_cap);
    float *out = p.scores + (size_t)g * p.c_cap + c0;
    if (c0 >= nc) {  // the whole tile is unused
        out[tid] = kNegInf;
        return;
    }
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    if (tid < D) {
        const T *q = reinterpret_cast<const T *>(p.q) + ((size_t)gc.b * p.Hq + gc.qh0) * D + tid;
        double s = 0.0;
        for (int h = 0; h < gc.nh; ++h) s += (double)to_f32(q[(size_t)h * D]);
        s_q[tid] = s;
    }
    __syncthreads();

    constexpr int DW = D / 4;
    const float *base = p.cent + (size_t)g * D * p.c_cap + c0 + 4 * lane;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 16
    for (int j = 0; j < DW; ++j) {
        const int d = wave * DW + j;
        const float4 v = *reinterpret_cast<const float4 *>(base + (size_t)d * p.c_cap);
        const double qq = s_q[d];
        a0 = fma((double)v.x, qq, a0);
        a1 = fma((double)v.y, qq, a1);
        a2 = fma((double)v.z, qq, a2);
        a3 = fma((double)v.w, qq, a3);
    }
    s_part[wave][4 * lane + 0] = a0;
    s_part[wave][4 * lane + 1] = a1;
    s_part[wave][4 * lane + 2] = a2;
    s_part[wave][4 * lane + 3] = a3;
    __syncthreads();
    const int c = c0 + tid;
    const double s = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    const bool ok = c < nc && p.size[(size_t)g * p.c_cap + c] > 0;
    out[tid] = ok ? (float)s : kNegInf;
    CKV_TMARK(1);
}

hipError_t launch_score(const ckv_kv *kv, const ckv_index *idx, const void *q, float *scores,
                        hipStream_t s) {
    const Window w = window_of(idx);
    ScoreParams p{q, idx->cent, idx->size, idx->n_comm, scores, idx->mode, kv->n_q_heads,
                  kv->n_kv_heads, idx->c_cap, w.first};
    const dim3 grid(idx->c_cap / 256, w.count);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    if (kv->head_dim == 128) {
        if (bf) CKV_LAUNCH((score_kernel<bf16_t, 128>), grid, dim3(256), s, p);
        else CKV_LAUNCH((score_kernel<float, 128>), grid, dim3(256), s, p);
    } else {
        if (bf) CKV_LAUNCH((score_kernel<bf16_t, 64>), grid, dim3(256), s, p);
        else CKV_LAUNCH((score_kernel<float, 64>), grid, dim3(256), s, p);
    }
    return hipGetLastError();
}

}  // namespace ckv
