// Edges, constant-time assignment and the O(d) centroid update (the
// CommunityKV page, Figure 1 panel (3): the top-kappa attended keys become the
// new token's edges and assign it to a community in constant time; Table 1:
// per-step update O(d); Table 6: sinks are excluded from the top-kappa pool).
//
// One 256-thread block per graph.  The edge weight of an attended non-sink
// token is its softmax probability (one head) or the sum of its heads'
// probabilities (query group).  With one head the logit orders the tokens the
// same way, so the logit itself is compared.  Each candidate becomes a 64-bit
// key (weight bits, then inverted position) so that one unsigned compare
// ranks it.  The kappa best keys are found without sorting all of them: a
// lower bound taken from the per-lane maxima leaves a few dozen candidates,
// which one wave orders exactly with repeated DPP max reductions.  Thread 0
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

// Edge candidate key: larger weight first, then lower position (0 = none).
__device__ __forceinline__ unsigned long long edge_key(float w, int pos) {
    if (w == 0.f) w = 0.f;  // one key for +0 and -0
    return ((unsigned long long)ordered_bits(w) << 32) | (0xFFFFFFFFu - (uint32_t)pos);
}

template <typename T, int D, int NH>
__global__ __launch_bounds__(256) void assign_kernel(AssignParams p) {
    __shared__ unsigned long long s_tau[4];
    __shared__ unsigned long long s_cand[64];
    __shared__ int s_ncand, s_ne;
    __shared__ int s_edges[CKV_MAX_KAPPA];
    __shared__ int s_elab[CKV_MAX_KAPPA];
    __shared__ int s_a, s_newsize;

    const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    CKV_TMARK(30);
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

    // Candidates as 64-bit keys, (order-preserving bits of the weight) << 32 |
    // ~position, so the larger key is the better edge (larger weight, then
    // lower position).  Up to kIpt per thread stay in registers.
    constexpr int kIpt = 24;
    unsigned long long ck[kIpt];
    const bool inreg = n <= kIpt * 256;
    {
        int cp[kIpt];
        float z[kIpt][NH];
#pragma unroll
        for (int i = 0; i < kIpt; ++i) {  // issue every load first
            const int j = tid + i * 256;
            const bool ok = inreg && j < n;
            cp[i] = ok ? tl[j] : -1;
#pragma unroll
            for (int h = 0; h < NH; ++h) z[i][h] = ok ? p.logits[((size_t)g * NH + h) * p.t_cap + j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kIpt; ++i) {
            float w;
            if constexpr (NH == 1) {
                w = z[i][0];
            } else {
                w = 0.f;
#pragma unroll
                for (int h = 0; h < NH; ++h) w += exp2f((z[i][h] - M[h]) * kLog2e) * Linv[h];
            }
            ck[i] = cp[i] >= p.n_sinks ? edge_key(w, cp[i]) : 0ull;
        }
    }

    CKV_TMARK(31);
    // Lower bound on the kappa-th best key: in each wave, the kappa-th largest
    // of the per-lane maxima (kappa keys of the wave reach it); the largest such
    // bound of the four waves still has kappa keys at or above it.
    const int kappa = p.kappa;
    unsigned long long tau = 0ull;
    if (inreg) {
        unsigned long long lm = 0ull;
#pragma unroll
        for (int i = 0; i < kIpt; ++i) lm = umax64(lm, ck[i]);
        unsigned long long tw = 0ull;
        int got = 0;
        for (int r = 0; r < kappa; ++r) {
            const unsigned long long m = wave_max_u64(lm);
            if (m == 0ull) break;
            if (lm == m) lm = 0ull;
            tw = m;
            ++got;
        }
        if (lane == 0) s_tau[wave] = got == kappa ? tw : 0ull;
        if (tid == 0) s_ncand = 0;
        __syncthreads();
        tau = umax64(umax64(s_tau[0], s_tau[1]), umax64(s_tau[2], s_tau[3]));
        if (tau != 0ull) {
#pragma unroll
            for (int i = 0; i < kIpt; ++i) {
                if (ck[i] >= tau) {
                    const int k = atomicAdd(&s_ncand, 1);
                    if (k < 64) s_cand[k] = ck[i];
                }
            }
        }
        __syncthreads();
    }
    CKV_TMARK(32);
    const bool fast = inreg && tau != 0ull && s_ncand <= 64;  // uniform

    int ne = 0;
    if (fast) {
        if (wave == 0) {  // exact order among the few candidates, one per lane
            unsigned long long c = lane < s_ncand ? s_cand[lane] : 0ull;
            for (int r = 0; r < kappa; ++r) {
                const unsigned long long m = wave_max_u64(c);
                if (m == 0ull) break;
                if (c == m) c = 0ull;
                if (lane == 0) s_edges[r] = (int)(0xFFFFFFFFu - (uint32_t)m);
                ++ne;
            }
        }
    } else if (wave == 0) {  // long token lists or degenerate weights: rounds over all tokens
        unsigned long long prev = ~0ull;
        for (int r = 0; r < kappa; ++r) {
            unsigned long long best = 0ull;
            for (int j = lane; j < n; j += 64) {
                const int pos = tl[j];
                if (pos < p.n_sinks) continue;
                const unsigned long long k = edge_key(weight(j), pos);
                if (k < prev && k > best) best = k;
            }
            best = wave_max_u64(best);
            if (best == 0ull) break;
            if (lane == 0) s_edges[r] = (int)(0xFFFFFFFFu - (uint32_t)best);
            prev = best;
            ++ne;
        }
    }
    if (wave == 0 && lane == 0) s_ne = ne;
    __syncthreads();
    ne = s_ne;
    CKV_TMARK(33);

    const int cap = min(p.l_cap, p.max_pages << p.ps_log2);
    const bool room = P < cap;
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

    CKV_TMARK(34);
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

    CKV_TMARK(35);
    // The last block advances every sequence with room by one token.  Every
    // block read seq_len before it counts itself in, so the increment cannot
    // race a read; the next kernel sees it across the kernel boundary.
    __syncthreads();
    if (tid == 0 && arrive_last(p.ctr, p.G)) {
        for (int bb = 0; bb < p.B; ++bb)
            if (p.seq_len[bb] < cap) p.seq_len[bb] += 1;
        reset_counter(p.ctr);
    }
    CKV_TMARK(36);
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
    if (kv->head_dim == DD && nh == NN) { CKV_LAUNCH((assign_kernel<TT, DD, NN>), grid, block, s, p); return hipGetLastError(); }
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
