// Centroid scoring (the CommunityKV page, Figure 1 panel (3): score the query
// against the community centroids; Table 1: retrieval is one pass over the
// centroids).
//
// This kernel computes screening scores from the int16 copy of the centroid
// table: s~[c] = cscale[c] * sum_d qbar_d * cq[d][c], with qbar rounded to
// float32 and a float32 sum.  Against the exact score (float64 sum of qbar_d
// times the float32 centroid, rounded to float32) the error is at most
// cscale[c] * |qbar|_1 * (1/2 + 32767 (D + 1) 2^-24 + ...) plus a few float32
// roundings of s~; the selection kernel turns that bound into intervals and
// computes the exact score of every community whose interval touches its
// budget cut, so the selection is the one the exact scores give.
//
// The screening copy is half the float32 table and streamed once from HBM, so
// the kernel is bandwidth-bound and runs on the vector units, not the matrix
// cores.  The table is stored transposed, [graph][dim][community], so lane j of
// a wave owns communities 4j..4j+3 of a 256-wide tile and every wave
// instruction reads 512 consecutive bytes of one dimension's row.  The four
// waves of a block split the dimensions and add their partial sums in a fixed
// order.  Empty communities and ids >= n_comm score -inf.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kScoreTile = 256;  // communities per block

struct ScoreParams {
    const void *q;
    const int16_t *cq;
    const float *cscale;
    const int32_t *size;
    const int32_t *n_comm;
    float *scores;
    int mode, Hq, Hkv, c_cap, g0, count;  // count: graphs in the launch window
};

// Signed 16-bit halves of a 32-bit word.
__device__ __forceinline__ float lo16(int w) { return (float)(int16_t)w; }
__device__ __forceinline__ float hi16(int w) { return (float)(w >> 16); }

template <typename T, int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
    __shared__ float s_q[D];
    __shared__ float s_part[4][kScoreTile];
    // Tile-major order: tile t of every graph of the window, then tile t + 1.
    // Workgroups go round-robin over the eight XCDs, so with a graph count
    // divisible by 8 all tiles of graph g run on the XCD that the selection
    // block of g (block g of its launch) runs on, and the scores, sizes and
    // scales it reads next are in that XCD's L2.
    const int tile = blockIdx.x / p.count, lg = blockIdx.x - tile * p.count;
    const int g = p.g0 + lg, c0 = tile * kScoreTile;
    CKV_TMARK(0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    // Every load of the block is issued before any is waited for, the query
    // first (it is needed first): one round trip instead of three.  c_cap %
    // 256 == 0, so every tile is whole and inside the table; a tile past the
    // graph's community count is read and then scored -inf like any unused id.
    // Query: the graph's heads (at most 8), loaded unconditionally at clamped
    // addresses so that no load waits for another.
    constexpr int kMaxHeads = 8;
    T qv[kMaxHeads];
    {
        const T *q = reinterpret_cast<const T *>(p.q) + ((size_t)gc.b * p.Hq + gc.qh0) * D + min(tid, D - 1);
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h) qv[h] = q[(size_t)min(h, gc.nh - 1) * D];
    }
    constexpr int DW = D / 4;
    const int16_t *base = p.cq + ((size_t)g * D + wave * DW) * p.c_cap + c0 + 4 * lane;
    int2 v[DW];
#pragma unroll
    for (int j = 0; j < DW; ++j) v[j] = *reinterpret_cast<const int2 *>(base + (size_t)j * p.c_cap);
    const int c = c0 + tid;  // kScoreTile == blockDim: one output per thread
    const int sz = p.size[(size_t)g * p.c_cap + c];
    const float scl = p.cscale[(size_t)g * p.c_cap + c];
    const int nc = min(p.n_comm[g], p.c_cap);
    if (tid < D) {  // the head sum in float64, heads in order
        double qs = 0.0;
#pragma unroll
        for (int h = 0; h < kMaxHeads; ++h)
            if (h < gc.nh) qs += (double)to_f32(qv[h]);
        s_q[tid] = (float)qs;
    }
    lds_barrier();

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < DW; ++j) {
        const float qq = s_q[wave * DW + j];
        acc[0] = fmaf(qq, lo16(v[j].x), acc[0]);
        acc[1] = fmaf(qq, hi16(v[j].x), acc[1]);
        acc[2] = fmaf(qq, lo16(v[j].y), acc[2]);
        acc[3] = fmaf(qq, hi16(v[j].y), acc[3]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) s_part[wave][4 * lane + k] = acc[k];
    lds_barrier();
    const float sum = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    p.scores[(size_t)g * p.c_cap + c] = (c < nc && sz > 0) ? scl * sum : kNegInf;
    CKV_TMARK(1);
}

hipError_t launch_score(const ckv_kv *kv, const ckv_index *idx, const void *q, float *scores,
                        hipStream_t s) {
    const Window w = window_of(idx);
    ScoreParams p{q, idx->cq, idx->cscale, idx->size, idx->n_comm, scores, idx->mode, kv->n_q_heads,
                  kv->n_kv_heads, idx->c_cap, w.first, w.count};
    const dim3 grid(ceil_div(idx->c_cap, kScoreTile) * w.count);
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
