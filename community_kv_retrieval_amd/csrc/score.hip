// Centroid scoring (the CommunityKV page, Figure 1 panel (3): score the query
// against the community centroids; Table 1: retrieval is one pass over the
// centroids).
//
// This kernel computes screening scores from the int8 copy of the centroid
// table: s~[c] = cscale[c] * sum_d qbar_d * cq[d][c], with qbar rounded to
// float32 and a float32 sum.  Against the exact score (float64 sum of qbar_d
// times the float32 centroid, rounded to float32) the error is at most
// cscale[c] * |qbar|_1 * (1/2 + (D + 4) 127 2^-24 + ...) plus a few float32
// roundings of s~; the selection kernel turns that bound into intervals and
// computes the exact score of every community whose interval touches its
// budget cut, so the selection is the one the exact scores give.
//
// The screening copy is a quarter of the float32 table and streamed once from
// HBM, so the kernel is bandwidth-bound and runs on the vector units, not the
// matrix cores.  The table is stored transposed and tile-major, [graph][tile
// of 256 communities][dim][256], so lane j of a wave owns communities 4j..4j+3
// of a tile, every wave instruction reads 256 consecutive bytes of one
// dimension's row, and a block streams one contiguous region.  The four
// waves of a block split the dimensions and add their partial sums in a fixed
// order.  Empty communities and ids >= n_comm score -inf.
//
// Each wave also hands the selection its candidates: of its 64 communities,
// the kCandPerWave with the largest upper bound U = s~ + E of the exact score
// (E the screening bound), with their bounds, sizes and base-member ranges,
// and the largest U among the ones it leaves out.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kScoreTile = 256;  // communities per block

struct ScoreParams {
    const void *q;
    const int8_t *cq;
    const float *cscale;
    const int32_t *size;
    const int32_t *n_comm;
    const int32_t *offs;
    float *scores;
    CandArrays cand;
    int mode, Hq, Hkv, c_cap, g0, count;  // count: graphs in the launch window
};

// Signed byte k of a 32-bit word.
template <int K>
__device__ __forceinline__ float byte8(int w) {
    return (float)((w << (24 - 8 * K)) >> 24);
}

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
    __builtin_amdgcn_sched_barrier(0);  // the query loads issue first
    constexpr int DW = D / 4;
    const int8_t *base = p.cq + cq_offset(g, wave * DW, c0, D, p.c_cap) + 4 * lane;
    int v[DW];
#pragma unroll
    for (int j = 0; j < DW; ++j)  // the codes are streamed once per step: nontemporal loads
        v[j] = __builtin_nontemporal_load(reinterpret_cast<const int *>(base + (size_t)j * 256));
    const int c = c0 + tid;  // kScoreTile == blockDim: one output per thread
    const int sz = p.size[(size_t)g * p.c_cap + c];
    const float scl = p.cscale[(size_t)g * p.c_cap + c];
    const int nc = min(p.n_comm[g], p.c_cap);
    // base members of c: offs[c] .. offs[c + 1] (the offsets row holds c_cap + 4 entries)
    const int32_t *orow = p.offs + (size_t)g * offs_stride(p.c_cap) + c;
    const int m0 = orow[0], m1 = orow[1];
    // The head sum in float64, heads in order, by every thread (threads past
    // D repeat the last dimension): kept unconditional, so that the query
    // loads stay ahead of the code loads and the sum waits for them alone.
    double qs = 0.0;
#pragma unroll
    for (int h = 0; h < kMaxHeads; ++h)
        if (h < gc.nh) qs += (double)to_f32(qv[h]);
    if (tid < D) s_q[tid] = (float)qs;
    lds_barrier();

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < DW; ++j) {
        const float qq = s_q[wave * DW + j];
        acc[0] = fmaf(qq, byte8<0>(v[j]), acc[0]);
        acc[1] = fmaf(qq, byte8<1>(v[j]), acc[1]);
        acc[2] = fmaf(qq, byte8<2>(v[j]), acc[2]);
        acc[3] = fmaf(qq, byte8<3>(v[j]), acc[3]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) s_part[wave][4 * lane + k] = acc[k];
    lds_barrier();
    const float sum = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
    const bool live = c < nc && sz > 0;
    const float sv = live ? scl * sum : kNegInf;
    p.scores[(size_t)g * p.c_cap + c] = sv;

    // Selection candidates of this wave's 64 communities: the kCandPerWave of
    // largest U = s~ + E (ties: lower lane), and the largest U left out.  The
    // kCandPerWave-th largest key is found bit by bit from the top (a count of
    // the lanes at or above each trial threshold), so no sort is needed.
    float qa = fabsf(s_q[lane]);
    if constexpr (D > 64) qa += fabsf(s_q[lane + 64]);
    const float kq = wave_sum_f(qa) * kScreenK;
    const float e = screen_bound(sv, scl, kq);
    const float up = sv + e, lw = sv - e;
    const uint32_t key = live ? ordered_bits(up) : 0u;
    uint32_t thr = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = thr | (1u << bit);
        const unsigned long long m = __ballot(key >= t);  // counted as two 32-bit halves: a scalar compare
        if (__builtin_popcount((uint32_t)m) + __builtin_popcount((uint32_t)(m >> 32)) >= kCandPerWave) thr = t;
    }
    const bool gt = live && key > thr, eq = live && key == thr;
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;  // lanes under this one
    const int ngt = __popcll(__ballot(gt));
    const bool take = gt || (eq && __popcll(__ballot(eq) & below) < kCandPerWave - ngt);
    const unsigned long long mt = __ballot(take);
    const int ntake = __popcll(mt);
    const float exv = wave_max_f(live && !take ? up : kNegInf);
    const int nw = p.cand.ncand / kCandPerWave;  // waves per graph
    const size_t cbase = (size_t)g * p.cand.ncand + ((size_t)tile * 4 + wave) * kCandPerWave;
    if (take) {
        const size_t k = cbase + __popcll(mt & below);
        p.cand.id[k] = c;
        p.cand.u[k] = up;
        p.cand.l[k] = lw;
        p.cand.sz[k] = sz;
        p.cand.o0[k] = m0;
        p.cand.len[k] = m1 - m0;
    }
    if (lane >= ntake && lane < kCandPerWave) p.cand.id[cbase + lane] = -1;
    if (lane == 0) p.cand.ex[(size_t)g * nw + tile * 4 + wave] = exv;
    CKV_TMARK(1);
}

hipError_t launch_score(const ckv_kv *kv, const ckv_index *idx, const void *q, float *scores,
                        const CandArrays &cand, hipStream_t s) {
    const Window w = window_of(idx);
    ScoreParams p{q, idx->cq, idx->cscale, idx->size, idx->n_comm, idx->offs, scores, cand, idx->mode,
                  kv->n_q_heads, kv->n_kv_heads, idx->c_cap, w.first, w.count};
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
