// Host-side declarations shared by the libckv translation units: launch
// shapes, workspace layout and the per-kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ckv.h"

namespace ckv {

// Tokens one gather block attends: 16 tokens per pass of its 256 threads
// (4 waves x 4 rows of 16 lanes), kGatherU passes per iteration, two
// iterations.  The workspace holds one partial record per head and span, and
// the assign kernel finds a deferred gather's records by the same span.
constexpr int kGatherU = 8;
constexpr int kGatherTokens = 16 * kGatherU * 2;
// The dense baseline: each block walks up to kDenseTokensMax consecutive
// tokens of one (sequence, kv head); dense_tokens() picks the span at launch.
constexpr int kDenseTokensMax = 2048;
constexpr int kDenseTokensMin = 512;

// Events armed by ckv_time_next_launch for the next step-kernel launch of
// this host thread.
struct LaunchTiming {
    hipEvent_t start, stop;
};
extern thread_local LaunchTiming g_next_timing;

inline LaunchTiming take_timing() {
    const LaunchTiming t = g_next_timing;
    g_next_timing = LaunchTiming{nullptr, nullptr};
    return t;
}

// Launches one step kernel, with the armed timing events if there are any.
#define CKV_LAUNCH(kernel, grid, block, stream, ...)                                             \
    do {                                                                                         \
        const ::ckv::LaunchTiming t_ = ::ckv::take_timing();                                     \
        if (t_.start)                                                                            \
            hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t_.start, t_.stop, 0, __VA_ARGS__); \
        else                                                                                     \
            hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                     \
    } while (0)

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
// Floats of one split-K partial record (accumulator, max, sum), padded to whole
// 128-byte cache lines so records written by different blocks never share a line.
constexpr int part_stride(int d) { return ((d + 2 + 31) / 32) * 32; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Row stride of the base CSR offsets (c_cap + 1 used, padded for 16-byte rows).
__host__ __device__ inline int offs_stride(int c_cap) { return c_cap + 4; }

// Centroid terms per partial record: the centroid-term kernel attends each
// group of kCentPerRecord of a graph's centroid terms in one block.
constexpr int kCentPerRecord = 16;
__host__ __device__ inline int cent_records(int n_cent) { return (n_cent + kCentPerRecord - 1) / kCentPerRecord; }

// Partial-record slots per graph and head of the gather: one per span of the
// longest list, and with a centroid budget one per kCentPerRecord centroid
// terms (written at the slots right after the graph's last span).
inline int gather_slots(const ckv_index *idx, int t_cap) {
    return ceil_div(t_cap > 0 ? t_cap : 1, kGatherTokens) + cent_records(idx->cent_budget);
}

// Graphs a step call processes: [first, first + count).
struct Window {
    int first, count;
};
inline Window window_of(const ckv_index *idx) {
    return idx->win_count > 0 ? Window{idx->win_first, idx->win_count} : Window{0, idx->n_graphs};
}

inline int group_of(const ckv_kv *kv) { return kv->n_q_heads / kv->n_kv_heads; }
inline int heads_per_graph(const ckv_kv *kv, const ckv_index *idx) {
    return idx->mode == CKV_MODE_PER_HEAD ? 1 : group_of(kv);
}
inline int ctx_cap(const ckv_kv *kv) { return kv->max_pages * kv->page_size; }

// Tokens per dense-baseline block: the longest of 2048, 1024 and 512 that
// still gives at least two blocks per CU (512 blocks) over the store's
// capacity, else 512.  Long spans amortise a block's start and records; short
// contexts need the blocks to fill the chip.
inline int dense_tokens(const ckv_kv *kv) {
    const long units = (long)kv->batch * kv->n_kv_heads;
    for (int t = kDenseTokensMax; t > kDenseTokensMin; t /= 2)
        if (units * ceil_div(ctx_cap(kv), t) >= 512) return t;
    return kDenseTokensMin;
}

// Workspace layout.  The dense baseline's region comes first and depends only
// on the K/V shape, so one workspace serves the dense baseline and the sparse
// path alike.  Counters are self-resetting.
struct WsLayout {
    size_t ctr_dense, part_dense;              // dense baseline
    size_t dense_total;                        // bytes the dense baseline needs
    size_t ctr_gather, ctr_assign;             // int32 counters (byte offsets)
    size_t cand, cand_end;                     // selection candidates (scoring -> selection)
    size_t part_gather;                        // float partials
    size_t build_cursor;                       // int32 [G][c_cap]
    size_t total;
};

// Selection candidates.  The scoring kernel keeps, of every wave's 64
// communities, the kCandPerWave of largest upper screening bound U, and the
// largest U it leaves out (at 128K about 2 communities per wave matter to the
// cut, so 15 are left out of the candidates only in degenerate cases); the selection works on those unless a left-out
// community could matter.  Per graph: (c_cap / 256) tiles x 4 waves x
// kCandPerWave records of (id, U, L, size, first base member, base members),
// id -1 for an empty slot, and one left-out maximum per wave.
constexpr int kCandPerWave = 15;
inline int cand_per_graph(int c_cap) { return c_cap / 256 * 4 * kCandPerWave; }
struct CandArrays {
    int32_t *id;
    float *u, *l;
    int32_t *sz, *o0, *len;
    float *ex;  // [G][ncand / kCandPerWave]
    int ncand;  // per graph
};
inline size_t cand_bytes(const ckv_index *idx) {
    const size_t n = (size_t)idx->n_graphs * cand_per_graph(idx->c_cap);
    return 6 * 4 * n + 4 * (n / kCandPerWave);
}

// idx == nullptr: only the dense baseline's part.
inline WsLayout ws_layout(const ckv_kv *kv, const ckv_index *idx, int t_cap) {
    WsLayout L{};
    const size_t units_dense = (size_t)kv->batch * kv->n_kv_heads;
    const size_t D2 = (size_t)part_stride(kv->head_dim);
    size_t off = 0;
    L.ctr_dense = off;
    off = align256(off + 4 * units_dense);
    L.part_dense = off;
    off += align256(4 * units_dense * group_of(kv) * (size_t)ceil_div(ctx_cap(kv), dense_tokens(kv)) * D2);
    L.dense_total = off;
    if (!idx) {
        L.total = off;
        return L;
    }
    const size_t G = (size_t)idx->n_graphs;
    L.ctr_gather = off;
    L.ctr_assign = off + 4 * G;
    off = align256(off + 4 * G + 4);
    L.cand = off;
    off += align256(cand_bytes(idx));
    L.cand_end = off;
    L.part_gather = off;
    off += align256(4 * G * heads_per_graph(kv, idx) * (size_t)gather_slots(idx, t_cap) * D2);
    L.build_cursor = off;
    off += align256(4 * G * (size_t)idx->c_cap);
    L.total = off;
    return L;
}

inline CandArrays cand_arrays(void *ws, const WsLayout &L, const ckv_index *idx) {
    CandArrays c;
    c.ncand = cand_per_graph(idx->c_cap);
    const size_t n = (size_t)idx->n_graphs * c.ncand;
    char *b = static_cast<char *>(ws) + L.cand;
    c.id = reinterpret_cast<int32_t *>(b);
    c.u = reinterpret_cast<float *>(c.id + n);
    c.l = c.u + n;
    c.sz = reinterpret_cast<int32_t *>(c.l + n);
    c.o0 = c.sz + n;
    c.len = c.o0 + n;
    c.ex = reinterpret_cast<float *>(c.len + n);
    return c;
}

// Launchers (each returns the hipError_t of its launches).
hipError_t launch_kv_write(const ckv_kv *kv, int b, int kh, int pos0, int n, const void *k,
                           const void *v, hipStream_t s);
hipError_t launch_index_build(const ckv_kv *kv, const ckv_index *idx, const int32_t *labels_in,
                              int32_t *cursor, hipStream_t s);
hipError_t launch_score(const ckv_kv *kv, const ckv_index *idx, const void *q, float *scores,
                        const CandArrays &cand, hipStream_t s);
hipError_t launch_select(const ckv_kv *kv, const ckv_index *idx, const void *q, const float *scores, int budget,
                         int max_comm, int t_cap, int32_t *sel, int32_t *sel_n, int32_t *top,
                         int32_t *tok_list, int32_t *tok_n, const CandArrays &cand, hipStream_t s);
hipError_t launch_gather(const ckv_kv *kv, const ckv_index *idx, const void *q,
                         const int32_t *tok_list, const int32_t *tok_n, int t_cap, float sm_scale,
                         float *out, float *logits, float *ml, float *part, int32_t *ctr,
                         hipStream_t s);
hipError_t launch_dense(const ckv_kv *kv, const void *q, float sm_scale, float *out, float *ml,
                        float *part, int32_t *ctr, hipStream_t s);
// Read-ceiling measurement: the gather's loads over given rows, XOR checksums.
hipError_t launch_read_rows(const ckv_kv *kv, const uint32_t *rows, int n, uint32_t *part, hipStream_t s);
// out != nullptr: the preceding gather was deferred; the assign kernel
// combines its partial records (part) into out and, if not null, ml.
hipError_t launch_assign(const ckv_kv *kv, const ckv_index *idx, const int32_t *tok_list,
                         const int32_t *tok_n, const float *logits, float *ml, int t_cap,
                         const int32_t *top, int kappa, const void *k_new, const void *v_new,
                         int32_t *edges, int32_t *assign, float *out, const float *part, int32_t *ctr,
                         hipStream_t s);

// Centroid budget: the communities whose centroids each graph's step attends
// (after the selection), and the softmax state of those centroid terms (into
// the gather's record slot after the graph's last span, before the gather).
hipError_t launch_centroid_select(const ckv_kv *kv, const ckv_index *idx, const void *q, const float *scores,
                                  const int32_t *sel, const int32_t *sel_n, hipStream_t s);
hipError_t launch_centroid_attend(const ckv_kv *kv, const ckv_index *idx, const void *q, const int32_t *tok_n,
                                  float sm_scale, float *part, int nslots, hipStream_t s);

// The gather with its partials and counters in the library's static scratch.
size_t noalloc_gather_bytes(const ckv_kv *kv, const ckv_index *idx, int t_cap);
hipError_t launch_gather_noalloc(const ckv_kv *kv, const ckv_index *idx, const void *q, const int32_t *tok_list,
                                 const int32_t *tok_n, int t_cap, float sm_scale, float *out, float *logits,
                                 float *ml, hipStream_t s);

// Attention-mass recall of every graph's heads from the gather's and the
// dense baseline's softmax states.
hipError_t launch_recall(const ckv_kv *kv, const ckv_index *idx, const float *ml, const float *dense_ml,
                         float *recall, hipStream_t s);

// Prefill graph construction of sequence b's first n positions.  lse: [Hq][n]
// floats of workspace (query-group mode).
hipError_t launch_prefill(const ckv_kv *kv, int mode, int b, const void *q, int n, int n_sinks, int kappa,
                          float sm_scale, int32_t *edges, float *weights, float *lse, hipStream_t s);

}  // namespace ckv
