// The C ABI of libckv: host-side argument validation, workspace carving and
// dispatch to the kernel launchers.  Validation runs before any HIP call, so
// every error return has enqueued nothing (and can be tested without a GPU).
#include <hip/hip_runtime.h>

#include "ckv.h"
#include "ckv_device.h"
#include "ckv_internal.h"

using namespace ckv;

namespace ckv {
thread_local LaunchTiming g_next_timing;
}

namespace {

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

ckv_status check_kv(const ckv_kv *kv) {
    if (!kv || !kv->kv || !kv->page_table || !kv->seq_len) return CKV_E_INVALID;
    if (kv->batch < 1 || kv->n_q_heads < 1 || kv->n_kv_heads < 1) return CKV_E_INVALID;
    if (kv->n_q_heads % kv->n_kv_heads) return CKV_E_INVALID;
    const int grp = kv->n_q_heads / kv->n_kv_heads;
    if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return CKV_E_UNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return CKV_E_UNSUPPORTED;
    if (kv->dtype != CKV_DTYPE_F32 && kv->dtype != CKV_DTYPE_BF16) return CKV_E_UNSUPPORTED;
    if (!pow2(kv->page_size) || kv->page_size > 1024) return CKV_E_INVALID;
    if (kv->max_pages < 1 || kv->n_pages < 1) return CKV_E_INVALID;
    if ((long long)kv->max_pages * kv->page_size > (1ll << 30)) return CKV_E_INVALID;
    // token rows of the pool must be addressable with 32-bit indices
    if ((long long)kv->n_pages * kv->n_kv_heads * kv->page_size > 0xFFFFFFFFll) return CKV_E_INVALID;
    if (kv->batch > 65535) return CKV_E_INVALID;
    return CKV_OK;
}

ckv_status check_index(const ckv_kv *kv, const ckv_index *idx) {
    if (!idx) return CKV_E_INVALID;
    if (idx->mode != CKV_MODE_PER_HEAD && idx->mode != CKV_MODE_QUERY_GROUP) return CKV_E_INVALID;
    const long long G = (long long)kv->batch * (idx->mode == CKV_MODE_PER_HEAD ? kv->n_q_heads : kv->n_kv_heads);
    if (idx->n_graphs != G || G > 65535) return CKV_E_INVALID;
    if (idx->c_cap < 256 || idx->c_cap % 256 || idx->c_cap > CKV_MAX_C_CAP) return CKV_E_INVALID;
    if (idx->l_cap < 1 || idx->tail_cap < 1 || idx->tail_cap > 4096 || idx->n_sinks < 0) return CKV_E_INVALID;
    if (!idx->n_comm || !idx->size || !idx->offs || !idx->toks || !idx->label || !idx->tail_pos ||
        !idx->tail_comm || !idx->tail_len || !idx->csum || !idx->cent || !idx->cq || !idx->cscale ||
        !idx->status)
        return CKV_E_INVALID;
    if (idx->cent_budget < 0 || idx->cent_budget > CKV_MAX_CENT) return CKV_E_INVALID;
    if (idx->cent_budget > 0 && (!idx->cent_sel || !idx->cent_n || !idx->vsum)) return CKV_E_INVALID;
    if (idx->win_count < 0 || idx->win_first < 0) return CKV_E_INVALID;
    if (idx->win_count == 0 ? idx->win_first != 0 : (long long)idx->win_first + idx->win_count > G)
        return CKV_E_INVALID;
    return CKV_OK;
}

ckv_status check_ws(const ckv_kv *kv, const ckv_index *idx, int t_cap, const void *ws, size_t bytes) {
    if (!ws || bytes < ws_layout(kv, idx, t_cap).total) return CKV_E_WORKSPACE;
    return CKV_OK;
}

ckv_status hip_status(hipError_t e) { return e == hipSuccess ? CKV_OK : CKV_E_HIP; }

char *at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

}  // namespace

extern "C" {

int32_t ckv_abi_version(void) { return 11; }

ckv_status ckv_time_next_launch(ckv_event_t start, ckv_event_t stop) {
    if ((start == nullptr) != (stop == nullptr)) return CKV_E_INVALID;
    g_next_timing = LaunchTiming{(hipEvent_t)start, (hipEvent_t)stop};
    return CKV_OK;
}

#ifdef CKV_PHASE_TRACE
// Profiling builds only: copy the 64 phase stamps to host memory.
int32_t ckv_trace_read(unsigned long long *host) {
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(ckv::g_phase_trace), sizeof(unsigned long long) * 64) ==
                   hipSuccess ? 0 : -1;
}

// Profiling builds only: copy the per-block stamps of the first n blocks
// (8 per block) to host memory, and clear them on the device.
int32_t ckv_block_trace_read(unsigned long long *host, int32_t n) {
    if (n < 0 || n > kBlockTraceBlocks) return -1;
    const size_t bytes = sizeof(unsigned long long) * 8 * (size_t)n;
    if (hipMemcpyFromSymbol(host, HIP_SYMBOL(ckv::g_block_trace), bytes) != hipSuccess) return -1;
    void *dev = nullptr;
    if (hipGetSymbolAddress(&dev, HIP_SYMBOL(ckv::g_block_trace)) != hipSuccess) return -1;
    return hipMemset(dev, 0, bytes) == hipSuccess ? 0 : -1;
}
#endif

const char *ckv_status_str(ckv_status s) {
    switch (s) {
        case CKV_OK: return "ok";
        case CKV_E_INVALID: return "invalid argument (null pointer, bad size or shape)";
        case CKV_E_UNSUPPORTED: return "unsupported head_dim, dtype or heads per group";
        case CKV_E_WORKSPACE: return "workspace missing or too small";
        case CKV_E_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

size_t ckv_workspace_bytes(const ckv_kv *kv, const ckv_index *idx, int32_t t_cap) {
    if (check_kv(kv) != CKV_OK || t_cap < 0) return 0;
    if (idx && check_index(kv, idx) != CKV_OK) return 0;
    return ws_layout(kv, idx, t_cap).total;
}

ckv_status ckv_kv_write(const ckv_kv *kv, int32_t b, int32_t kv_head, int32_t pos0, int32_t n,
                        const void *k, const void *v, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if (b < 0 || b >= kv->batch || kv_head < 0 || kv_head >= kv->n_kv_heads || pos0 < 0 || n < 0 ||
        (long long)pos0 + n > (long long)kv->max_pages * kv->page_size)
        return CKV_E_INVALID;
    if (n == 0) return CKV_OK;
    if (!k || !v) return CKV_E_INVALID;
    return hip_status(launch_kv_write(kv, b, kv_head, pos0, n, k, v, (hipStream_t)stream));
}

ckv_status ckv_index_build(const ckv_kv *kv, const ckv_index *idx, const int32_t *labels_in,
                           void *ws, size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!labels_in) return CKV_E_INVALID;
    if ((st = check_ws(kv, idx, 0, ws, ws_bytes)) != CKV_OK) return st;
    const WsLayout L = ws_layout(kv, idx, 0);
    return hip_status(launch_index_build(kv, idx, labels_in, (int32_t *)at(ws, L.build_cursor),
                                         (hipStream_t)stream));
}

ckv_status ckv_score_centroids(const ckv_kv *kv, const ckv_index *idx, const void *q, float *scores,
                               void *ws, size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!q || !scores) return CKV_E_INVALID;
    const WsLayout L = ws_layout(kv, idx, 0);
    if (!ws || ws_bytes < L.total) return CKV_E_WORKSPACE;
    return hip_status(launch_score(kv, idx, q, scores, cand_arrays(ws, L, idx), (hipStream_t)stream));
}

ckv_status ckv_select_communities(const ckv_kv *kv, const ckv_index *idx, const void *q,
                                  const float *scores, int32_t budget, int32_t max_comm, int32_t t_cap,
                                  int32_t *sel, int32_t *sel_n, int32_t *top, int32_t *tok_list,
                                  int32_t *tok_n, void *ws, size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!q || !scores || !sel || !sel_n || !top || !tok_list || !tok_n) return CKV_E_INVALID;
    if (budget < 0 || max_comm < 0) return CKV_E_INVALID;
    const long long need = (long long)idx->n_sinks + (budget < idx->l_cap ? budget : idx->l_cap);
    if (t_cap < need) return CKV_E_INVALID;
    const WsLayout L = ws_layout(kv, idx, 0);
    if (!ws || ws_bytes < L.total) return CKV_E_WORKSPACE;
    hipError_t e = launch_select(kv, idx, q, scores, budget, max_comm, t_cap, sel, sel_n, top, tok_list, tok_n,
                                 cand_arrays(ws, L, idx), (hipStream_t)stream);
    if (e == hipSuccess && idx->cent_budget > 0)
        e = launch_centroid_select(kv, idx, q, scores, sel, sel_n, (hipStream_t)stream);
    return hip_status(e);
}

ckv_status ckv_gather_attend(const ckv_kv *kv, const ckv_index *idx, const void *q,
                             const int32_t *tok_list, const int32_t *tok_n, int32_t t_cap,
                             float sm_scale, float *out, float *logits, float *ml, void *ws,
                             size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!q || !tok_list || !tok_n || !logits) return CKV_E_INVALID;
    if ((out == nullptr) != (ml == nullptr)) return CKV_E_INVALID;  // both (complete) or neither (deferred)
    if (t_cap < 1) return CKV_E_INVALID;
    if ((st = check_ws(kv, idx, t_cap, ws, ws_bytes)) != CKV_OK) return st;
    const WsLayout L = ws_layout(kv, idx, t_cap);
    return hip_status(launch_gather(kv, idx, q, tok_list, tok_n, t_cap, sm_scale, out, logits, ml,
                                    (float *)at(ws, L.part_gather), (int32_t *)at(ws, L.ctr_gather),
                                    (hipStream_t)stream));
}

ckv_status ckv_gather_attend_noalloc(const ckv_kv *kv, const ckv_index *idx, const void *q,
                                     const int32_t *tok_list, const int32_t *tok_n, int32_t t_cap,
                                     float sm_scale, float *out, float *logits, float *ml,
                                     ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!q || !tok_list || !tok_n || !logits || !out || !ml) return CKV_E_INVALID;
    if (t_cap < 1) return CKV_E_INVALID;
    if (noalloc_gather_bytes(kv, idx, t_cap) > CKV_NOALLOC_SCRATCH_BYTES) return CKV_E_WORKSPACE;
    return hip_status(launch_gather_noalloc(kv, idx, q, tok_list, tok_n, t_cap, sm_scale, out, logits, ml,
                                            (hipStream_t)stream));
}

ckv_status ckv_assign_update(const ckv_kv *kv, const ckv_index *idx, const int32_t *tok_list,
                             const int32_t *tok_n, const float *logits, float *ml, int32_t t_cap,
                             const int32_t *top, int32_t kappa, const void *k_new, const void *v_new,
                             int32_t *edges, int32_t *assign, float *out, void *ws, size_t ws_bytes,
                             ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!tok_list || !tok_n || !logits || !top || !k_new || !v_new || !edges || !assign)
        return CKV_E_INVALID;
    if (!out && !ml) return CKV_E_INVALID;  // a complete gather's softmax state is read
    if (kappa < 1 || kappa > CKV_MAX_KAPPA || t_cap < 1) return CKV_E_INVALID;
    if ((st = check_ws(kv, idx, t_cap, ws, ws_bytes)) != CKV_OK) return st;
    const WsLayout L = ws_layout(kv, idx, t_cap);
    return hip_status(launch_assign(kv, idx, tok_list, tok_n, logits, ml, t_cap, top, kappa, k_new, v_new,
                                    edges, assign, out, (const float *)at(ws, L.part_gather),
                                    (int32_t *)at(ws, L.ctr_assign), (hipStream_t)stream));
}

ckv_status ckv_dense_attend(const ckv_kv *kv, const void *q, float sm_scale, float *out, float *ml,
                            void *ws, size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if (!q || !out) return CKV_E_INVALID;
    const WsLayout L = ws_layout(kv, nullptr, 0);
    if (!ws || ws_bytes < L.dense_total) return CKV_E_WORKSPACE;
    return hip_status(launch_dense(kv, q, sm_scale, out, ml, (float *)at(ws, L.part_dense),
                                   (int32_t *)at(ws, L.ctr_dense), (hipStream_t)stream));
}

ckv_status ckv_attention_recall(const ckv_kv *kv, const ckv_index *idx, const float *ml, const float *dense_ml,
                                float *recall, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if ((st = check_index(kv, idx)) != CKV_OK) return st;
    if (!ml || !dense_ml || !recall) return CKV_E_INVALID;
    return hip_status(launch_recall(kv, idx, ml, dense_ml, recall, (hipStream_t)stream));
}

ckv_status ckv_read_rows(const ckv_kv *kv, const uint32_t *rows, int32_t n, uint32_t *part, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if (n < 0) return CKV_E_INVALID;
    if (n == 0) return CKV_OK;  // nothing to read, nothing launched
    if (!rows || !part) return CKV_E_INVALID;
    return hip_status(launch_read_rows(kv, rows, n, part, (hipStream_t)stream));
}

size_t ckv_prefill_workspace_bytes(const ckv_kv *kv, int32_t mode, int32_t n) {
    if (check_kv(kv) != CKV_OK || n < 1) return 0;
    if (mode != CKV_MODE_PER_HEAD && mode != CKV_MODE_QUERY_GROUP) return 0;
    return align256((size_t)4 * kv->n_q_heads * n);
}

ckv_status ckv_prefill_topk(const ckv_kv *kv, int32_t mode, int32_t b, const void *q, int32_t n,
                            int32_t n_sinks, int32_t kappa, float sm_scale, int32_t *edges, float *weights,
                            void *ws, size_t ws_bytes, ckv_stream_t stream) {
    ckv_status st = check_kv(kv);
    if (st != CKV_OK) return st;
    if (kv->dtype != CKV_DTYPE_BF16) return CKV_E_UNSUPPORTED;  // matrix cores take bf16 operands
    if (mode != CKV_MODE_PER_HEAD && mode != CKV_MODE_QUERY_GROUP) return CKV_E_INVALID;
    if (!q || !edges || b < 0 || b >= kv->batch) return CKV_E_INVALID;
    if (n < 1 || (int64_t)n > (int64_t)kv->max_pages * kv->page_size) return CKV_E_INVALID;
    if (n_sinks < 0 || kappa < 1 || kappa > CKV_MAX_KAPPA || !(sm_scale > 0.f)) return CKV_E_INVALID;
    if (mode == CKV_MODE_QUERY_GROUP) {
        const int grp = kv->n_q_heads / kv->n_kv_heads;
        if (grp > 4 || kappa > 16) return CKV_E_UNSUPPORTED;
    }
    const size_t need = ckv_prefill_workspace_bytes(kv, mode, n);
    if (!ws || ws_bytes < need) return CKV_E_WORKSPACE;
    return hip_status(launch_prefill(kv, mode, b, q, n, n_sinks, kappa, sm_scale, edges, weights, (float *)ws,
                                     (hipStream_t)stream));
}

}  // extern "C"
