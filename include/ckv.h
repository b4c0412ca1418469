/*
 * ckv.h -- C ABI of libckv.so, the CommunityKV sparse decode step on AMD
 * MI355X (gfx950).
 *
 * The method: "CommunityKV: Efficient Long-Context Decoding via Graph
 * Partitioning" (McKenna, Alexandridis, Susanj, Liu).  Its Figure 1 caption,
 * panel (3), the incremental update, describes one decode step.  The query is
 * compared with every community's centroid.  The best communities are
 * gathered within a token budget.  Softmax attention over their tokens and
 * the sink tokens is computed exactly.  The kappa tokens that attention
 * weights most become the new token's edges, and they decide its community
 * at a cost independent of the context length.  Table 1 gives the per-step
 * update as O(d).  Table 6 fixes kappa = 8, sinks excluded from the
 * top-kappa pool, and one graph per query head as the default; Tables 5 and 6
 * name query-group graphs (one graph per kv head, shared by its query heads)
 * as the alternative aggregation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers inside the descriptors and all array arguments are DEVICE
 *    pointers (memory the caller allocated on the GPU the stream belongs to),
 *    except the descriptors themselves, which are host structs read during
 *    the call only, and the two host calls ckv_leiden_partition and
 *    ckv_partition_quality, whose arrays are host memory.
 *  - The library allocates, frees and synchronises nothing.  Every call only
 *    validates its arguments on the host and enqueues kernels on `stream`
 *    (NULL = the null stream); it returns before the work runs.  Buffers must
 *    stay alive until the stream work has finished.
 *  - Host-side validation happens before any device call: a call that returns
 *    an error has enqueued nothing.
 *  - Outputs are overwritten, never accumulated.  Results are deterministic
 *    (no floating-point atomics; every reduction has a fixed order).
 *  - Conditions only the device can see (a full tail, a position beyond the
 *    capacity, a bad label) set bits in idx->status[0]; they never fault.
 *  - Calls that touch disjoint descriptors and workspaces may run on different
 *    streams concurrently.  Two calls sharing a workspace must be ordered.
 *
 * Memory layout
 * -------------
 *  K/V pool: kv->kv holds n_pages pages; page p, kv head h, slot s holds one
 *    token as [K row | V row], each head_dim elements of kv->dtype:
 *      element (p, h, s, which, e) at ((((p * n_kv_heads + h) * page_size + s) * 2 + which) * head_dim + e)
 *    which = 0 for K, 1 for V.  Position t of sequence b lives in page
 *    page_table[b * max_pages + t / page_size], slot t % page_size.
 *  Graphs: one per query head (CKV_MODE_PER_HEAD, G = batch * n_q_heads,
 *    graph g = b * n_q_heads + qh, indexing kv head qh / (n_q_heads/n_kv_heads))
 *    or one per kv head (CKV_MODE_QUERY_GROUP, G = batch * n_kv_heads,
 *    graph g = b * n_kv_heads + kh, read by query heads kh*grp .. kh*grp+grp-1).
 *  Positions 0 .. n_sinks-1 of every sequence are sink tokens: attended at
 *    every step, in no community, never an edge.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *ckv_stream_t; /* a hipStream_t */
struct ihipEvent_t;
typedef struct ihipEvent_t *ckv_event_t;   /* a hipEvent_t */

typedef int32_t ckv_status;
#define CKV_OK             0
#define CKV_E_INVALID     -1 /* null pointer, bad size or shape */
#define CKV_E_UNSUPPORTED -2 /* head_dim not 64/128, unknown dtype, heads per group not 1/2/4/8 */
#define CKV_E_WORKSPACE   -3 /* workspace missing or smaller than ckv_workspace_bytes() */
#define CKV_E_HIP         -4 /* a kernel launch failed (the HIP error is consumed) */

/* bits of idx->status[0] (set by the device, cleared by ckv_index_build) */
#define CKV_ST_TAIL_FULL   1 /* a new token found its graph's tail full: left unassigned */
#define CKV_ST_CAPACITY    2 /* a new position reached l_cap or the page table's end: not stored */
#define CKV_ST_BAD_LABEL   4 /* ckv_index_build met a label >= n_comm[g] (ignored) */

#define CKV_DTYPE_F32  0
#define CKV_DTYPE_BF16 1

#define CKV_MODE_PER_HEAD    0
#define CKV_MODE_QUERY_GROUP 1

#define CKV_MAX_KAPPA 32
#define CKV_MAX_C_CAP 16384
#define CKV_MAX_CENT  256   /* largest centroid budget (Table 6 ablates 0, 4, 16, 64, 256) */
/* Static device scratch of ckv_gather_attend_noalloc (bytes, per GPU). */
#define CKV_NOALLOC_SCRATCH_BYTES (4u << 20)

/* The paged K/V store of one attention layer (layout above). */
typedef struct ckv_kv {
    void          *kv;          /* [n_pages][n_kv_heads][page_size][2][head_dim] of dtype */
    const int32_t *page_table;  /* [batch][max_pages] page ids, each < n_pages */
    int32_t       *seq_len;     /* [batch] tokens cached per sequence; ckv_assign_update adds one */
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;         /* n_q_heads / n_kv_heads must be 1, 2, 4 or 8 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t page_size;          /* power of two, 1 .. 1024 */
    int32_t max_pages;          /* page-table entries per sequence */
    int32_t n_pages;
    int32_t dtype;              /* CKV_DTYPE_F32 or CKV_DTYPE_BF16 (also the dtype of q, k_new, v_new) */
} ckv_kv;

/* Community state of every graph of one layer.  Community ids of graph g are
 * 0 .. n_comm[g]-1.  Members of community c are the base members
 * toks[g][offs[g][c] .. offs[g][c+1]) (fixed by ckv_index_build) plus the
 * tokens appended since, listed in the graph's tail. */
typedef struct ckv_index {
    int32_t  mode;       /* CKV_MODE_PER_HEAD or CKV_MODE_QUERY_GROUP */
    int32_t  n_graphs;   /* G: batch*n_q_heads (per head) or batch*n_kv_heads (group) */
    int32_t  c_cap;      /* community slots per graph: multiple of 256, <= CKV_MAX_C_CAP */
    int32_t  l_cap;      /* positions per graph (label stride); new positions must stay below */
    int32_t  tail_cap;   /* tokens a graph can take after the build, 1 .. 4096 */
    int32_t  n_sinks;    /* leading sink positions, >= 0 */
    int32_t *n_comm;     /* [G] communities in use, <= c_cap (set by the caller before the build) */
    int32_t *size;       /* [G][c_cap] members per community (base + tail) */
    int32_t *offs;       /* [G][c_cap+4] base CSR offsets into toks: entries 0..c_cap used, rows
                            padded to c_cap+4 so that every row starts 16-byte aligned */
    int32_t *toks;       /* [G][l_cap] base members, grouped by community, ascending position */
    int32_t *label;      /* [G][l_cap] community of every position, -1 = sink / none */
    int32_t *tail_pos;   /* [G][tail_cap] appended positions, in order */
    int32_t *tail_comm;  /* [G][tail_cap] their communities */
    int32_t *tail_len;   /* [G] */
    double  *csum;       /* [G][c_cap][head_dim] exact float64 key sum of every community */
    float   *cent;       /* [G][c_cap][head_dim] centroid = float32(csum / size), one row per community */
    int8_t  *cq;         /* [G][c_cap / 256][head_dim][256] screening copy of cent, tile-major
                            (element (g, d, c) at ((g * c_cap/256 + c/256) * head_dim + d) * 256
                            + c % 256): cent ~ cscale * cq, cq = round(cent / cscale) in
                            [-127, 127] */
    float   *cscale;     /* [G][c_cap] max_d |cent[d]| / 127 of every community (0: zero column) */
    int32_t *status;     /* [1] CKV_ST_* bits */
    /* Launch window of the four step calls (score, select, gather, assign):
     * they process graphs win_first .. win_first + win_count - 1 only
     * (win_count = 0: every graph; win_first must then be 0).  Windows let a
     * caller run disjoint sets of graphs on different streams so that one set's
     * latency-bound calls overlap another set's bandwidth-bound ones.  Every
     * array stays indexed by the global graph id, so windows never share a slot.
     * Within one decode step the ckv_assign_update windows must cover every
     * graph exactly once: seq_len advances when the last of the G graphs is done.
     * ckv_index_build and ckv_dense_attend ignore the window. */
    int32_t  win_first;
    int32_t  win_count;
    /* Centroid budget (Table 6, "Centroid Budget"; 0, the default, turns it
     * off and the four arrays below may be NULL).  With cent_budget = N in
     * 1 .. CKV_MAX_CENT the attention of each step also takes the centroids of
     * the N best-ranked non-empty communities that the selection did not take
     * (all of them when fewer are left): each is one softmax term with key
     * mu_c = float32(csum[c] / size[c]) (the stored centroid), value
     * float32(vsum[c] / size[c]) (the members' mean value) and logit
     * sm_scale * q . mu_c + ln size[c], i.e. the mass of size[c] tokens whose
     * key is the centroid.  Centroid terms never become edges, but their mass
     * is part of the normaliser of every token's probability (and of ml). */
    int32_t  cent_budget;
    int32_t *cent_sel;   /* [G][cent_budget] those communities, ascending ids (ckv_select_communities) */
    int32_t *cent_n;     /* [G] their count */
    double  *vsum;       /* [G][c_cap][head_dim] exact float64 value sum of every community
                            (ckv_index_build, ckv_assign_update) */
} ckv_index;

/* Bytes of workspace the calls below need for this layer shape and a token
 * list capacity t_cap.  The workspace must be zero-filled once before its first
 * use; the calls leave it zero-filled where it matters.  0 on bad arguments. */
size_t ckv_workspace_bytes(const ckv_kv *kv, const ckv_index *idx, int32_t t_cap);

/* Store n tokens of sequence b, kv head kv_head at positions pos0 .. pos0+n-1.
 * k, v: [n][head_dim] of kv->dtype.  Does not change seq_len (setup helper for
 * filling a prefill cache). */
ckv_status ckv_kv_write(const ckv_kv *kv, int32_t b, int32_t kv_head, int32_t pos0, int32_t n,
                        const void *k, const void *v, ckv_stream_t stream);

/* Build the community index from a given partition (the page's prefill
 * partition, Figure 1 panel (2); here any labelling the caller supplies).
 * labels_in: [G][l_cap] community of each position < seq_len[b] (-1 = none;
 * positions < n_sinks are always sinks).  idx->n_comm must hold each graph's
 * community count.  Fills size, offs, toks, label, csum, cent (the centroid
 * is the mean of the members' keys; Figure 1 panel (2) draws one per
 * community) and its screening copy cq/cscale, empties the tails and clears
 * status.  With a centroid budget it also fills vsum, the members' value sums. */
ckv_status ckv_index_build(const ckv_kv *kv, const ckv_index *idx, const int32_t *labels_in,
                           void *ws, size_t ws_bytes, ckv_stream_t stream);

/* Screening scores of every community against the query (Figure 1 panel (3):
 * the query is scored against the community centroids).  q:
 * [batch][n_q_heads][head_dim] of kv->dtype.  The graph's query qbar is its
 * head's q (per head) or the sum of its group's q (query group; the group's
 * summed q . centroid).  The exact score of community c is
 * float32(sum_d qbar_d * cent[d][c]) with the sum in float64; this call writes
 * scores[G][c_cap] = cscale[c] * sum_d float32(qbar_d) * cq(d, c) (float32),
 * within cscale[c] * |qbar|_1 * 0.51 + 2^-20 |score| of the exact score, and
 * -inf for empty communities and ids >= n_comm[g].  ckv_select_communities
 * resolves the ranking exactly from these bounds.  It also leaves in ws the
 * selection's candidates (of every 64 consecutive communities the 16 of
 * largest upper bound, and the largest bound left out), which the next
 * ckv_select_communities on the same ws reads: ws must hold at least
 * ckv_workspace_bytes(kv, idx, 0) bytes (CKV_E_WORKSPACE otherwise). */
ckv_status ckv_score_centroids(const ckv_kv *kv, const ckv_index *idx, const void *q,
                               float *scores, void *ws, size_t ws_bytes, ckv_stream_t stream);

/* Retrieve communities under the token budget (Figure 1 panel (3): a subset
 * of the communities is retrieved; Tables 2-3: the subset is bounded by a
 * token budget).  Communities are ranked by their exact score (see
 * ckv_score_centroids), higher first, ties to the lower id; the longest prefix
 * of that ranking whose member count stays within `budget` (and, if
 * max_comm > 0, holds at most max_comm communities) is taken: the first
 * community that does not fit ends the walk.  `scores` are the screening
 * scores of ckv_score_centroids for the same q; exact scores are computed here
 * (from the centroid rows idx->cent) for every community whose screening
 * interval leaves its place relative to the cut open, so the result is that of
 * the exact scores.
 * Outputs per graph: sel[G][c_cap] taken ids ascending, sel_n[G] their count,
 * top[G] the best-ranked non-empty community (-1 if none), tok_list[G][t_cap]
 * the attended positions (sinks first, then members of the taken communities)
 * and tok_n[G] their count.  Requires t_cap >= n_sinks + min(budget, l_cap).
 * ws: the workspace the preceding ckv_score_centroids for the same q wrote its
 * candidates to (at least ckv_workspace_bytes(kv, idx, 0) bytes).  The
 * selection works on the candidates when they provably hold every community
 * the result depends on, and on every community otherwise; the result is the
 * same either way.  With idx->cent_budget > 0 a second kernel then writes
 * idx->cent_sel and idx->cent_n: the cent_budget best-ranked non-empty
 * communities outside sel, ranked by exact score as above. */
ckv_status ckv_select_communities(const ckv_kv *kv, const ckv_index *idx, const void *q,
                                  const float *scores, int32_t budget, int32_t max_comm, int32_t t_cap,
                                  int32_t *sel, int32_t *sel_n, int32_t *top,
                                  int32_t *tok_list, int32_t *tok_n, void *ws, size_t ws_bytes,
                                  ckv_stream_t stream);

/* Exact softmax attention of each graph's query heads over its token list
 * (Figure 1 panel (3): attention over the retrieved subset is exact and also
 * covers the sink tokens).  z_j = sm_scale * q . k_j in float32 from the stored K; outputs:
 * out[batch][n_q_heads][head_dim] float32 (every query head is written),
 * logits[G][hpg][t_cap] the z_j of each slot < tok_n[g] (hpg = heads per graph),
 * ml[G][hpg][2] = (max z, sum exp(z - max)).  The list is split into spans of
 * 256 tokens attended in parallel; their softmax states are combined in span
 * order (log-sum-exp).
 * Deferred combine: with out == NULL and ml == NULL the call writes the logits
 * and leaves the per-span states in ws; the next ckv_assign_update on the same
 * ws, tok_list, tok_n and t_cap with a non-NULL out then writes out and ml,
 * bit for bit as this call would have (the combine then overlaps the assign's
 * own work instead of ending the gather).  Exactly one of out, ml NULL:
 * CKV_E_INVALID.
 * With idx->cent_budget > 0 the call first attends each graph's centroid
 * terms (idx->cent_sel, idx->cent_n) in a kernel of its own, which leaves one
 * more softmax state per head for every 16 terms, after the spans' (up to
 * ceil(t_cap / 256) + ceil(cent_budget / 16) states per head in all); the
 * combine takes them last, and out and ml cover tokens and centroid terms
 * alike. */
ckv_status ckv_gather_attend(const ckv_kv *kv, const ckv_index *idx, const void *q,
                             const int32_t *tok_list, const int32_t *tok_n, int32_t t_cap,
                             float sm_scale, float *out, float *logits, float *ml,
                             void *ws, size_t ws_bytes, ckv_stream_t stream);

/* ckv_gather_attend without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as ckv_gather_attend
 * in its complete mode (out and ml required, bit-identical outputs), but the
 * split-K partial records and arrival counters live in a static device array
 * of the library, CKV_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends; the call allocates nothing.  The scratch need is 256-aligned
 * 4 * n_graphs bytes of counters plus 4 * n_graphs * heads_per_graph *
 * nspan * (32 * ceil((head_dim + 2) / 32)) bytes of records, nspan =
 * ceil(t_cap / 256) + ceil(cent_budget / 16); a
 * larger need returns CKV_E_WORKSPACE before anything is enqueued.  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  The
 * stream must belong to the current device.  Each call clears its counters
 * with a small fill kernel before the gather, so it may be captured and
 * replayed.  Errors as for ckv_gather_attend; out == NULL or ml == NULL:
 * CKV_E_INVALID. */
ckv_status ckv_gather_attend_noalloc(const ckv_kv *kv, const ckv_index *idx, const void *q,
                                     const int32_t *tok_list, const int32_t *tok_n, int32_t t_cap,
                                     float sm_scale, float *out, float *logits, float *ml,
                                     ckv_stream_t stream);

/* Edges, assignment and update (Figure 1 panel (3): the kappa keys the new
 * token attends to most become its edges and decide its community, at a cost
 * independent of the context length; Table 1: per-step update O(d)).  For every graph: the kappa
 * non-sink attended tokens of largest weight (per head: the head's attention
 * probability; query group: the sum of its heads' probabilities), ties to the
 * lower position, become edges[G][kappa] (-1 padded); the new token goes to the
 * community holding most edges, ties to the lowest id (top[g] if there is no
 * edge): assign[G].  Then, at P = seq_len[b]: label[P] = a, P joins a's tail,
 * size[a] += 1, csum[a] += k_new, cent[a] = float32(csum[a] / size[a]) (and
 * vsum[a] += v_new with a centroid budget); k_new,
 * v_new ([batch][n_kv_heads][head_dim] of kv->dtype) are stored at P, and
 * finally seq_len[b] += 1.
 * out == NULL: the gather was complete and its ml (required) is read.
 * out != NULL: the preceding ckv_gather_attend was deferred (out == ml == NULL
 * there); this call first completes it, writing out[batch][n_q_heads][head_dim]
 * and, when ml is not NULL, ml[G][hpg][2], from the states left in ws, and
 * takes the weights from those same states. */
ckv_status ckv_assign_update(const ckv_kv *kv, const ckv_index *idx, const int32_t *tok_list,
                             const int32_t *tok_n, const float *logits, float *ml,
                             int32_t t_cap, const int32_t *top, int32_t kappa,
                             const void *k_new, const void *v_new, int32_t *edges,
                             int32_t *assign, float *out, void *ws, size_t ws_bytes,
                             ckv_stream_t stream);

/* Dense flash-decode baseline: softmax attention of every query head over all
 * seq_len[b] cached tokens of its kv head.  out[batch][n_q_heads][head_dim];
 * ml (NULL: not written) [batch][n_q_heads][2] = (max z, sum exp(z - max)) of
 * every head over all its tokens.  With the ml of ckv_gather_attend for the
 * same q, ckv_attention_recall gives the share of the dense attention mass
 * that the attended tokens carry (the page's attention-mass recall, Figure 3). */
ckv_status ckv_dense_attend(const ckv_kv *kv, const void *q, float sm_scale, float *out, float *ml,
                            void *ws, size_t ws_bytes, ckv_stream_t stream);

/* Attention-mass recall (Figure 3: the share of the full attention mass that
 * the retrieved tokens capture), for every graph and head:
 *   recall[G][hpg] = exp(m_T - m) * l_T / l
 * from (m_T, l_T) = ml[G][hpg][2] of ckv_gather_attend (a complete gather, or
 * the ml a deferred gather's ckv_assign_update wrote) and (m, l) =
 * dense_ml[batch][n_q_heads][2] of ckv_dense_attend on the same q and cache
 * state: the softmax mass of the attended tokens over that of every cached
 * token.  Evaluated in float64, stored as float32; 0 where the graph attended
 * nothing (l_T = 0).  With a centroid budget the gather's ml also holds the
 * centroid terms' mass, so the value is then the share of the attended
 * tokens and the centroid terms together.  All three arrays are device
 * memory.  Processes every graph (the launch window is ignored).  Errors: CKV_E_INVALID for a NULL
 * array or a bad descriptor. */
ckv_status ckv_attention_recall(const ckv_kv *kv, const ckv_index *idx, const float *ml, const float *dense_ml,
                                float *recall, ckv_stream_t stream);

/* Prefill graph construction (Figure 1 panel (1): during prefill each query is
 * linked to the keys it attends to most; sinks are left out of the pool, Table 6;
 * Table 10 times it as the fused top-kappa selection).  For every position
 * i < n of sequence b and every graph g of the sequence (per head: query head
 * g, g < n_q_heads; query group: kv head g, g < n_kv_heads) the kappa keys
 * j with n_sinks <= j < i of largest weight, ties to the lower position,
 * become edges[g][i][0..kappa) in rank order (-1 padded when fewer).  The
 * weight of key j is the causal softmax probability of query i over keys
 * 0..i (the token itself included in the normaliser, not in the pool) with
 * logits sm_scale * q . k: the head's own (per head) or the sum over the
 * group's heads (query group).  weights (NULL: not written) [g][i][kappa]
 * holds those weights, 0 for padding.  Logits are float32 products of the
 * bf16 operands (matrix cores), the weights float32.
 * q: [n][n_q_heads][head_dim] bf16 (the prompt's queries); keys: positions
 * 0..n-1 of sequence b in the store (written beforehand, e.g. by
 * ckv_kv_write; seq_len is neither read nor changed).  Requires a bf16 store
 * (else CKV_E_UNSUPPORTED), 1 <= kappa <= 32, sm_scale > 0; query groups need
 * at most 4 heads per group and kappa <= 16 (else CKV_E_UNSUPPORTED).  ws:
 * ckv_prefill_workspace_bytes(kv, mode, n) bytes (holds the per-head
 * log-sum-exp of the group mode). */
size_t ckv_prefill_workspace_bytes(const ckv_kv *kv, int32_t mode, int32_t n);
ckv_status ckv_prefill_topk(const ckv_kv *kv, int32_t mode, int32_t b, const void *q, int32_t n,
                            int32_t n_sinks, int32_t kappa, float sm_scale, int32_t *edges, float *weights,
                            void *ws, size_t ws_bytes, ckv_stream_t stream);

/* Leiden partition of token graphs (Figure 1 panel (2): the prefill graph is
 * partitioned with the Leiden algorithm; Figure 2: a resolution parameter
 * gamma sets the community size; Tables 8 and 9: re-partitioning the grown
 * graph, "Refresh", against incremental assignment).  HOST call: every
 * pointer below is host memory, and nothing is enqueued on a GPU; Figure 4
 * runs the partitioning beside the GPU, asynchronously, which a caller gets
 * by running this call on a thread of its own.
 *
 * Graph g (0 <= g < n_graphs) has n_tokens[g] tokens.  Row i of
 * edges[g][row_stride][kappa] (int32) lists token i's edges (-1 = none), as
 * ckv_prefill_topk writes them for prompt tokens and ckv_assign_update for
 * decoded ones; rows >= n_tokens[g] are not read.  The graph's nodes are the
 * tokens n_sinks .. n_tokens[g]-1; each listed edge i -> j adds one to the
 * weight between i and j (so 1 or 2).  An edge to a sink, to itself or to a
 * token >= n_tokens[g] is an error.
 *
 * Quality is modularity at resolution gamma_num / gamma_den; every decision
 * compares exact integers.  The algorithm (Traag, Waltman and van Eck, Sci.
 * Rep. 9, 5233, 2019): fast local moving, refinement into well-connected
 * sub-communities, aggregation, until every community of a level is one node;
 * its random choices are fixed (queue in token order; the best community wins,
 * staying on ties, the lower id among equal ones; a new community only when
 * strictly better; refinement takes the best strictly positive merge), so the
 * result depends on the graph alone.
 *
 * Outputs: labels[g][row_stride] = community of each token, numbered 0, 1, ...
 * in order of first token, -1 for sinks and rows >= n_tokens[g]; n_comm[g];
 * quality[g] (NULL: not written) = modularity Q of the result.  n_threads
 * host threads share the graphs (0: one per hardware thread).
 * Errors (CKV_E_INVALID, outputs then undefined): n_graphs < 0, NULL arrays,
 * kappa outside 1..32, n_tokens[g] outside 0..row_stride, gamma_num < 0,
 * gamma_den <= 0, a bad edge, or a graph so large that (2m)^2 * 4 *
 * max(gamma_num, gamma_den) reaches 2^62. */
ckv_status ckv_leiden_partition(int32_t n_graphs, const int32_t *n_tokens, int32_t n_sinks, const int32_t *edges,
                                int64_t row_stride, int32_t kappa, int64_t gamma_num, int64_t gamma_den,
                                int32_t n_threads, int32_t *labels, int32_t *n_comm, double *quality);

/* Tokens decoded while a partition was computed join it (HOST call, host
 * pointers; Figure 4 runs the partitioning beside the model, Figure 1 panel
 * (3) places a new token by its edges).  For every graph g, tokens
 * first[g] .. n_tokens[g]-1 of labels[g][row_stride] are set in increasing
 * order: each joins the community most of its edges' targets (rows of
 * edges[g][row_stride][kappa], as for ckv_leiden_partition) are in, ties to
 * the lower id, targets without a community (-1) not voting; a token with no
 * such target starts community n_comm[g], which then grows by one.  labels
 * below first[g] are read, not written; n_comm[g] is read and updated.
 * Errors (CKV_E_INVALID, nothing written): n_graphs < 0, NULL arrays, kappa
 * outside 1..32, first[g] outside 0..n_tokens[g], n_tokens[g] > row_stride,
 * n_comm[g] < 0, or an edge of a token to itself or a later token. */
ckv_status ckv_extend_partition(int32_t n_graphs, const int32_t *first, const int32_t *n_tokens, const int32_t *edges,
                                int64_t row_stride, int32_t kappa, int32_t *labels, int32_t *n_comm);

/* Modularity Q (Figure 3, left) of given labels on the same token graphs as
 * ckv_leiden_partition (HOST call, host pointers, same edge rules): labels of
 * tokens n_sinks .. n_tokens[g]-1 must lie in 0 .. n_tokens[g]-n_sinks-1 (any
 * numbering, e.g. the labels an index holds after incremental assignment);
 * quality[g] is written.  Q = 0 for a graph without edges.  Errors as above,
 * plus CKV_E_INVALID for a label out of range. */
ckv_status ckv_partition_quality(int32_t n_graphs, const int32_t *n_tokens, int32_t n_sinks, const int32_t *edges,
                                 int64_t row_stride, int32_t kappa, int64_t gamma_num, int64_t gamma_den,
                                 int32_t n_threads, const int32_t *labels, double *quality);

/* Read ceiling of the gather's access pattern, for measurement (no part of
 * the method).  Reads the K|V rows rows[0..n) of the store (row id r: token
 * slot r % page_size of kv head (r / page_size) % n_kv_heads of page
 * r / (page_size * n_kv_heads), i.e. the record at kv + r * 2 * head_dim
 * elements) with the gather's loads: 256 rows per block, 16 lanes per row.
 * part[ceil(n / 256)] (device, uint32) receives, per block of 256 rows, the
 * XOR of every 32-bit word of those rows, so a caller can check that all bytes
 * were read.  Row ids at or past n_pages * n_kv_heads * page_size are clamped
 * to the last row.  n == 0: nothing is launched.  Errors: CKV_E_INVALID for
 * n < 0 or a NULL rows / part with n > 0. */
ckv_status ckv_read_rows(const ckv_kv *kv, const uint32_t *rows, int32_t n, uint32_t *part, ckv_stream_t stream);

/* Kernel timing for profiling harnesses (no part of the method).  Arms the
 * calling host thread so that the next kernel launched by one of
 * ckv_score_centroids, ckv_select_communities, ckv_gather_attend,
 * ckv_assign_update, ckv_dense_attend, ckv_read_rows (each launches exactly one
 * kernel without a centroid budget; with one, select and gather time their
 * main kernel, not the centroid kernel) or
 * ckv_prefill_topk (one kernel per head; the query-group mode launches two and
 * the pair times the first) has `start` and `stop` recorded by its own dispatch (hipExtLaunchKernel):
 * hipEventElapsedTime(start, stop) is then that kernel's execution time, with
 * no marker packets around it.  One-shot: the launch consumes the pair.  A call
 * that fails validation launches nothing and leaves the pair armed.  Both
 * events must come from hipEventCreate (timing enabled) on the call's device;
 * start == stop == NULL disarms.  Not for use under stream capture.
 * Returns CKV_E_INVALID when exactly one of the two is NULL. */
ckv_status ckv_time_next_launch(ckv_event_t start, ckv_event_t stop);

/* Static description of a status code. */
const char *ckv_status_str(ckv_status s);

/* Library ABI version (bumped when a signature or layout changes). */
int32_t ckv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CKV_H */
