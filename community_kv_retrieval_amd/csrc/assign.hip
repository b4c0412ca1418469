// Edges, constant-time assignment and the O(d) centroid update (the
// CommunityKV page, Figure 1 panel (3): the top-kappa attended keys become the
// new token's edges and assign it to a community in constant time; Table 1:
// per-step update O(d); Table 6: sinks are excluded from the top-kappa pool).
//
// One 256-thread block per graph.  The edge weight of an attended non-sink
// token is its softmax probability (one head) or the sum of its heads'
// probabilities (query group).  With one head the logit orders the tokens the
// same way, so the logit itself is compared.  The kappa best tokens (larger
// weight first, lower position on ties) are extracted one per round: each
// round every thread proposes its best token ranked strictly below the
// previous winner and a block reduction picks the best proposal.  Thread 0
// takes the majority label of the edges (lowest id on ties), then the block
// appends the token to that community: label, tail entry, member count, the
// exact float64 key sum and the float32 centroid column.  Graphs that own the
// kv head store the new key and value; the last block to finish advances every
// sequence length.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

struct AssignParams {
    void *kv;
    const int32_t *page_table;
    int32_t *seq_len;
    int B, Hq, Hkv, ps_log2, max_pages;
    int mode, G, c_cap, l_cap, tail_cap, n_sinks, t_cap, kappa;
    int32_t *size;
    int32_t *label;
    int32_t *tail_pos;
    int32_t *tail_comm;
    int32_t *tail_len;
    double *csum;
    float *cent;
    int32_t *status;
    const int32_t *tok_list;
    const int32_t *tok_n;
    const float *logits;
    const float *ml;
    const int32_t *top;
    const void *k_new;
    const void *v_new;
    int32_t *edges;
    int32_t *assign;
    int32_t *ctr;
};

__device__ __forceinline__ bool better(float w1, int p1, float w2, int p2) {
    return w1 > w2 || (w1 == w2 && p1 < p2);
}

template <typename T, int D, int NH>
__global__ __launch_bounds__(256) void assign_kernel(AssignParams p) {
    __shared__ float s_rw[4];
    __shared__ int s_rp[4];
    __shared__ int s_edges[CKV_MAX_KAPPA];
    __shared__ int s_elab[CKV_MAX_KAPPA];
    __shared__ int s_a, s_newsize;

    const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int P = p.seq_len[gc.b];
    const int n = p.tok_n[g];
    const int32_t *tl = p.tok_list + (size_t)g * p.t_cap;

    float M[NH], Linv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        M[h] = p.ml[((size_t)g * NH + h) * 2];
        Linv[h] = 1.f / p.ml[((size_t)g * NH + h) * 2 + 1];
    }
    auto weight = [&](int j) -> float {
        if constexpr (NH == 1) {
            return p.logits[(size_t)g * p.t_cap + j];
        } else {
            float w = 0.f;
#pragma unroll
            for (int h = 0; h < NH; ++h)
                w += exp2f((p.logits[((size_t)g * NH + h) * p.t_cap + j] - M[h]) * kLog2e) * Linv[h];
            return w;
        }
    };

    // Candidate weights, computed once.  Up to kIpt per thread stay in
    // registers; longer token lists re-read them from memory every round.
    constexpr int kIpt = 24;
    float cw[kIpt];
    int cp[kIpt];
    const bool inreg = n <= kIpt * 256;
    {
        // issue every load first, then compute the weights
        float z[kIpt][NH];
#pragma unroll
        for (int i = 0; i < kIpt; ++i) {
            const int j = tid + i * 256;
            const bool ok = inreg && j < n;
            cp[i] = ok ? tl[j] : 0x7fffffff;
#pragma unroll
            for (int h = 0; h < NH; ++h) z[i][h] = ok ? p.logits[((size_t)g * NH + h) * p.t_cap + j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kIpt; ++i) {
            if (cp[i] == 0x7fffffff || cp[i] < p.n_sinks) {
                cp[i] = 0x7fffffff;
                cw[i] = kNegInf;
            } else if constexpr (NH == 1) {
                cw[i] = z[i][0];
            } else {
                float w = 0.f;
#pragma unroll
                for (int h = 0; h < NH; ++h) w += exp2f((z[i][h] - M[h]) * kLog2e) * Linv[h];
                cw[i] = w;
            }
        }
    }

    float pw = __builtin_huge_valf();
    int pp = -1;
    int ne = 0;
    for (int r = 0; r < p.kappa; ++r) {
        float bw = kNegInf;
        int bp = 0x7fffffff;
        if (inreg) {
#pragma unroll
            for (int i = 0; i < kIpt; ++i) {
                if (cp[i] != 0x7fffffff && better(pw, pp, cw[i], cp[i]) && better(cw[i], cp[i], bw, bp)) {
                    bw = cw[i];
                    bp = cp[i];
                }
            }
        } else {
            for (int j = tid; j < n; j += 256) {
                const int pos = tl[j];
                if (pos < p.n_sinks) continue;
                const float w = weight(j);
                if (better(pw, pp, w, pos) && better(w, pos, bw, bp)) {
                    bw = w;
                    bp = pos;
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ow = __shfl_xor(bw, o, 64);
            const int op = __shfl_xor(bp, o, 64);
            if (better(ow, op, bw, bp)) {
                bw = ow;
                bp = op;
            }
        }
        if (lane == 0) {
            s_rw[wave] = bw;
            s_rp[wave] = bp;
        }
        __syncthreads();
        {
            float w = s_rw[0];
            int q = s_rp[0];
#pragma unroll
            for (int i = 1; i < 4; ++i)
                if (better(s_rw[i], s_rp[i], w, q)) {
                    w = s_rw[i];
                    q = s_rp[i];
                }
            pw = w;
            pp = q;
        }
        __syncthreads();
        if (pp == 0x7fffffff) break;
        if (tid == 0) s_edges[r] = pp;
        ++ne;
    }

    const int cap = min(p.l_cap, p.max_pages << p.ps_log2);
    const bool room = P < cap;
    __syncthreads();  // s_edges complete
    if (tid < ne) s_elab[tid] = p.label[(size_t)g * p.l_cap + s_edges[tid]];
    const int tn = p.tail_len[g];
    __syncthreads();
    if (tid == 0) {
        int best = -1, bestc = 0;
        for (int r = 0; r < ne; ++r) {
            const int c = s_elab[r];
            if (c < 0) continue;
            int k = 0;
            for (int r2 = 0; r2 < ne; ++r2) k += (s_elab[r2] == c);
            if (k > bestc || (k == bestc && c < best)) {
                best = c;
                bestc = k;
            }
        }
        const int a = best >= 0 ? best : p.top[g];
        for (int r = 0; r < p.kappa; ++r) p.edges[(size_t)g * p.kappa + r] = r < ne ? s_edges[r] : -1;
        p.assign[g] = a;
        int joined = -1;
        if (!room) {
            atomicOr(p.status, CKV_ST_CAPACITY);
        } else if (a >= 0) {
            if (tn < p.tail_cap) {
                p.label[(size_t)g * p.l_cap + P] = a;
                p.tail_pos[(size_t)g * p.tail_cap + tn] = P;
                p.tail_comm[(size_t)g * p.tail_cap + tn] = a;
                p.tail_len[g] = tn + 1;
                s_newsize = p.size[(size_t)g * p.c_cap + a] + 1;
                p.size[(size_t)g * p.c_cap + a] = s_newsize;
                joined = a;
            } else {
                atomicOr(p.status, CKV_ST_TAIL_FULL);
                p.label[(size_t)g * p.l_cap + P] = -1;
            }
        } else {
            p.label[(size_t)g * p.l_cap + P] = -1;
        }
        s_a = joined;
    }
    __syncthreads();

    const T *kn = reinterpret_cast<const T *>(p.k_new) + ((size_t)gc.b * p.Hkv + gc.kh) * D;
    const T *vn = reinterpret_cast<const T *>(p.v_new) + ((size_t)gc.b * p.Hkv + gc.kh) * D;
    const int a = s_a;
    if (a >= 0 && tid < D) {
        const size_t ci = ((size_t)g * p.c_cap + a) * D + tid;
        const double cs = p.csum[ci] + (double)to_f32(kn[tid]);
        p.csum[ci] = cs;
        p.cent[((size_t)g * D + tid) * p.c_cap + a] = (float)(cs / (double)s_newsize);
    }
    // The graph of the group's first query head stores the new key and value.
    const bool owner = p.mode == CKV_MODE_QUERY_GROUP || (gc.qh0 % (p.Hq / p.Hkv)) == 0;
    if (owner && room) {
        const int page = p.page_table[(size_t)gc.b * p.max_pages + (P >> p.ps_log2)];
        T *row = reinterpret_cast<T *>(p.kv) +
                 ((((size_t)page * p.Hkv + gc.kh) << p.ps_log2) | (size_t)(P & ((1 << p.ps_log2) - 1))) * (2 * D);
        for (int i = tid; i < 2 * D; i += 256) row[i] = i < D ? kn[i] : vn[i - D];
    }

    // The last block advances every sequence with room by one token.  Every
    // block read seq_len before it counts itself in, so the increment cannot
    // race a read; the next kernel sees it across the kernel boundary.
    __syncthreads();
    if (tid == 0 && arrive_last(p.ctr, p.G)) {
        for (int bb = 0; bb < p.B; ++bb)
            if (p.seq_len[bb] < cap) p.seq_len[bb] += 1;
        reset_counter(p.ctr);
    }
}

hipError_t launch_assign(const ckv_kv *kv, const ckv_index *idx, const int32_t *tok_list,
                         const int32_t *tok_n, const float *logits, const float *ml, int t_cap,
                         const int32_t *top, int kappa, const void *k_new, const void *v_new,
                         int32_t *edges, int32_t *assign, int32_t *ctr, hipStream_t s) {
    AssignParams p{};
    p.kv = kv->kv;
    p.page_table = kv->page_table;
    p.seq_len = kv->seq_len;
    p.B = kv->batch;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    p.max_pages = kv->max_pages;
    p.mode = idx->mode;
    p.G = idx->n_graphs;
    p.c_cap = idx->c_cap;
    p.l_cap = idx->l_cap;
    p.tail_cap = idx->tail_cap;
    p.n_sinks = idx->n_sinks;
    p.t_cap = t_cap;
    p.kappa = kappa;
    p.size = idx->size;
    p.label = idx->label;
    p.tail_pos = idx->tail_pos;
    p.tail_comm = idx->tail_comm;
    p.tail_len = idx->tail_len;
    p.csum = idx->csum;
    p.cent = idx->cent;
    p.status = idx->status;
    p.tok_list = tok_list;
    p.tok_n = tok_n;
    p.logits = logits;
    p.ml = ml;
    p.top = top;
    p.k_new = k_new;
    p.v_new = v_new;
    p.edges = edges;
    p.assign = assign;
    p.ctr = ctr;
    const int nh = heads_per_graph(kv, idx);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    const dim3 grid(idx->n_graphs), block(256);
#define CKV_AS(TT, DD, NN) \
    if (kv->head_dim == DD && nh == NN) { hipLaunchKernelGGL((assign_kernel<TT, DD, NN>), grid, block, 0, s, p); return hipGetLastError(); }
#define CKV_AS_T(TT) \
    CKV_AS(TT, 64, 1) CKV_AS(TT, 64, 2) CKV_AS(TT, 64, 4) CKV_AS(TT, 64, 8) \
    CKV_AS(TT, 128, 1) CKV_AS(TT, 128, 2) CKV_AS(TT, 128, 4) CKV_AS(TT, 128, 8)
    if (bf) {
        CKV_AS_T(bf16_t)
    } else {
        CKV_AS_T(float)
    }
#undef CKV_AS_T
#undef CKV_AS
    return hipErrorInvalidValue;
}

}  // namespace ckv
