// Edges, assignment and the O(d) centroid update (the CommunityKV page,
// Figure 1 panel (3): the keys the new token attends to most become its edges
// and decide its community at a cost independent of the context length;
// Table 1: per-step update O(d); Table 6: sinks never become edges).
//
// One 256-thread block per graph.  The edge weight of an attended non-sink
// token is its softmax probability (one head) or the sum of its heads'
// probabilities (query group).  With one head the logit orders the tokens the
// same way, so the logit itself is compared.  Each candidate becomes a 64-bit
// key (weight bits, then inverted position) so that one unsigned compare
// ranks it.  The kappa best keys are found without sorting all of them: a
// lower bound taken from the per-lane maxima leaves a few dozen candidates,
// each of which finds its exact rank by counting the better ones.  One wave
// takes the majority label of the edges (lowest id on ties), then the block
// appends the token to that community: label, tail entry, member count, the
// exact float64 key sum and the float32 centroid column.  Graphs that own the
// kv head store the new key and value.  Each block counts itself in as soon as
// it has read its sequence length; the last to count in advances every
// sequence length at its end.
#include "ckv_device.h"
#include "ckv_internal.h"
#include "combine.h"

namespace ckv {

struct AssignParams {
    void *kv;
    const int32_t *page_table;
    int32_t *seq_len;
    int B, Hq, Hkv, ps_log2, max_pages;
    int mode, G, g0, c_cap, l_cap, tail_cap, n_sinks, t_cap, kappa;
    int32_t *size;
    int32_t *label;
    int32_t *tail_pos;
    int32_t *tail_comm;
    int32_t *tail_len;
    double *csum;
    float *cent;
    int8_t *cq;
    float *cscale;
    int32_t *status;
    const int32_t *tok_list;
    const int32_t *tok_n;
    const float *logits;
    float *ml;           // read (gather complete) or written (deferred combine)
    float *out;          // not null: combine the deferred gather's records into out
    const float *part;   // the gather's partial records
    int nchunk;          // gather record slots per graph and head
    const int32_t *cent_n;  // centroid budget: centroid terms per graph (their records follow the spans')
    double *vsum;        // centroid budget: value sums (else null)
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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    return wave_reduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// How the kernel gets the attention's softmax state.  Complete: the gather
// wrote ml.  Deferred: the gather left per-span records that this kernel
// combines (into out and ml); with at most kPreChunks spans and four heads the
// accumulators are loaded with the first round trip (DeferRegs), otherwise
// when they are combined (Defer).
enum AssignMode { kAssignComplete = 0, kAssignDeferRegs = 1, kAssignDefer = 2 };
constexpr int kLenLds = 64;  // sequences whose lengths the first round trip reads
constexpr int kPreChunks = 20;

template <typename T, int D, int NH, int MODE>
__global__ __launch_bounds__(256) void assign_kernel(AssignParams p) {
    constexpr int kIpt = 18;  // list entries per thread held in registers (4 608 per graph)
    __shared__ unsigned long long s_cand[64];
    __shared__ uint32_t s_tau[4];
    __shared__ int s_ncand, s_ne, s_a;
    __shared__ int s_edges[CKV_MAX_KAPPA];
    __shared__ int s_elab[CKV_MAX_KAPPA];
    __shared__ float s_max[4];
    __shared__ CombineLds<NH> s_comb;
    __shared__ int s_P;                      // the graph's sequence length (position of the new token)
    __shared__ int s_len[kLenLds];           // every sequence's length, for the advance at the end
    constexpr int PS = part_stride(D);

    const int g = p.g0 + blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr bool defer = MODE != kAssignComplete;
    constexpr bool regs = MODE == kAssignDeferRegs;
    static_assert(!regs || NH <= 4, "preloaded combine: at most four heads");
    CKV_TMARK(30);
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int32_t *tl = p.tok_list + (size_t)g * p.t_cap;
    // Everything this block reads first, issued together: nothing here waits
    // for the token count (the list and the logits are t_cap long; entries at
    // or past tok_n are masked afterwards).
    const int n = p.tok_n[g];
    // Sequence lengths: wave 0 only (the others take P from LDS below).
    const bool few = p.B <= kLenLds;  // uniform
    int P0 = 0, len_l = 0;
    if (wave == 0) {
        P0 = p.seq_len[gc.b];
        if (few) len_l = p.seq_len[min(lane, p.B - 1)];
    }
    const int tn = p.tail_len[g];
    const int topc = p.top[g];
    float M[NH], Linv[NH];
    if constexpr (!defer) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            M[h] = NH > 1 ? p.ml[((size_t)g * NH + h) * 2] : 0.f;
            Linv[h] = NH > 1 ? 1.f / p.ml[((size_t)g * NH + h) * 2 + 1] : 0.f;
        }
    }
    // Deferred gather: nact records per head hold this graph's spans, and
    // then its centroid terms' records.
    const float *PR = p.part + (size_t)g * NH * p.nchunk * PS;
    const int nact = (n > 0 ? (n + kGatherTokens - 1) / kGatherTokens : 0) +
                     ((defer && p.cent_n) ? cent_records(p.cent_n[g]) : 0);
    const int jmax = min(p.t_cap, kIpt * 256);
    int cp[kIpt];
    float z[kIpt][NH];
#pragma unroll
    for (int i = 0; i < kIpt; ++i) {
        const int j = tid + i * 256;
        const bool ok = j < jmax;
        cp[i] = ok ? tl[j] : -1;
#pragma unroll
        for (int h = 0; h < NH; ++h) z[i][h] = ok ? p.logits[((size_t)g * NH + h) * p.t_cap + j] : 0.f;
    }
    // DeferRegs: then the records of every span the list can have, with no
    // condition on any load (clamped addresses), so that the LDS write of the
    // (max, sum) pairs waits for them and nothing after them: the
    // accumulators stay in flight until waves 1-3 combine them while wave 0
    // ranks the edges.
    float st_m = 0.f, st_l = 0.f;
    float ov[combine_pairs<D, NH, 192>()][regs ? kPreChunks : 1];
    if constexpr (regs) {
        const float *r = PR + (size_t)min(tid, NH * p.nchunk - 1) * PS;  // head / chunk = tid div / mod nchunk
        st_m = r[D];
        st_l = r[D + 1];
        combine_preload_all<D, NH, PS, 192, kPreChunks>(PR, p.nchunk, tid - 64, ov);
    }
    if (tid == 0) s_ncand = 0;
    if constexpr (regs) {
        if (tid < NH * p.nchunk) {
            const int h = tid / p.nchunk;
            s_comb.m[h][tid - h * p.nchunk] = st_m;
            s_comb.l[h][tid - h * p.nchunk] = st_l;
        }
    } else if constexpr (defer) {
        combine_stage<NH, D, PS, false>(PR, p.nchunk, nact, s_comb);
    }

    // The block counts itself in as soon as wave 0 holds the lengths (the
    // asm takes them as inputs, so their loads have returned, and no memory
    // access moves across it): every thread takes P from LDS, so once every
    // block of the step has counted in, every read of seq_len is done and the
    // last block may advance the lengths, at its end, without a round trip
    // there.
    bool last = false;
    if (wave == 0) {
        asm volatile("" ::"v"(P0), "v"(len_l) : "memory");
        if (few && lane < p.B) s_len[lane] = len_l;
        if (tid == 0) {
            s_P = P0;
            last = arrive_last(p.ctr, p.G);
        }
    }
    const int cap = min(p.l_cap, p.max_pages << p.ps_log2);
    const bool owner = p.mode == CKV_MODE_QUERY_GROUP || (gc.qh0 % (p.Hq / p.Hkv)) == 0;
    const T *kn = reinterpret_cast<const T *>(p.k_new) + ((size_t)gc.b * p.Hkv + gc.kh) * D;
    const T *vn = reinterpret_cast<const T *>(p.v_new) + ((size_t)gc.b * p.Hkv + gc.kh) * D;

    // Deferred gather: every head's softmax state (M, L) from the records, by
    // the combine's own steps, so the weights below equal those computed from
    // a complete gather's ml.  The barriers up to the ranking order LDS
    // traffic only: the accumulator loads above stay in flight.
    if constexpr (defer) {
        lds_barrier();
        if (nact >= 1 && nact <= kCombineLds) combine_heads<NH>(nact, s_comb);
        lds_barrier();
        if constexpr (NH > 1) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float L = 1.f;
                M[h] = kNegInf;
                if (nact >= 1 && nact <= kCombineLds) {
                    M[h] = s_comb.M[h];
                    L = s_comb.L[h];
                } else if (nact > kCombineLds) {
                    head_state_long<D, PS, false>(PR, p.nchunk, nact, h, M[h], L);
                }
                Linv[h] = 1.f / L;
            }
        }
    }

    // Candidates as 64-bit keys, (order-preserving bits of the weight) << 32 |
    // ~position, so the larger key is the better edge (larger weight, then
    // lower position).  With one head the logit orders the tokens as the
    // probability does.
    const bool inreg = n <= kIpt * 256;  // uniform
    unsigned long long ck[kIpt];
#pragma unroll
    for (int i = 0; i < kIpt; ++i) {
        const int j = tid + i * 256;
        float w;
        if constexpr (NH == 1) {
            w = z[i][0];
        } else {
            w = 0.f;
#pragma unroll
            for (int h = 0; h < NH; ++h) w += exp2f((z[i][h] - M[h]) * kLog2e) * Linv[h];
        }
        ck[i] = (inreg && j < n && cp[i] >= p.n_sinks) ? edge_key(w, cp[i]) : 0ull;
    }
    CKV_TMARK(31);

    // Lower bound on the kappa-th best weight: in each wave, kappa rounds of
    // the largest remaining per-lane maximum (every round retires at least one
    // lane, so kappa keys of the wave reach the last value); the largest bound
    // of the four waves still has kappa keys at or above it.  No wave with
    // kappa candidates: every candidate is kept.
    const int kappa = p.kappa;
    if (inreg) {
        uint32_t lm = 0u;
#pragma unroll
        for (int i = 0; i < kIpt; ++i) lm = max(lm, (uint32_t)(ck[i] >> 32));
        uint32_t tw = 0u;
        int got = 0;
        for (int r = 0; r < kappa; ++r) {
            const uint32_t m = wave_max_u32(lm);
            if (m == 0u) break;
            if (lm == m) lm = 0u;
            tw = m;
            ++got;
        }
        if (lane == 0) s_tau[wave] = got == kappa ? tw : 0u;
        lds_barrier();
        uint32_t tau = max(max(s_tau[0], s_tau[1]), max(s_tau[2], s_tau[3]));
        if (tau == 0u) tau = 1u;
#pragma unroll
        for (int i = 0; i < kIpt; ++i) {
            if (ck[i] != 0ull && (uint32_t)(ck[i] >> 32) >= tau) {
                const int k = atomicAdd(&s_ncand, 1);
                if (k < 64) s_cand[k] = ck[i];
            }
        }
        lds_barrier();
    }
    CKV_TMARK(32);
    const int ncand = inreg ? s_ncand : 65;
    const bool fast = ncand <= 64;  // uniform

    if (fast) {
        if (wave == 0) {
            // Each candidate counts the better ones: its rank.  Its label load
            // is in flight meanwhile.
            const unsigned long long mine = lane < ncand ? s_cand[lane] : 0ull;
            const int pos = (int)(0xFFFFFFFFu - (uint32_t)mine);
            const int lab = lane < ncand ? p.label[(size_t)g * p.l_cap + pos] : -1;
            int rank = 0;
            for (int k0 = 0; k0 < ncand; k0 += 8) {  // k0 + 7 < 64: reads stay inside s_cand
                unsigned long long kk[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) kk[u] = s_cand[k0 + u];
#pragma unroll
                for (int u = 0; u < 8; ++u) rank += (k0 + u < ncand && kk[u] > mine) ? 1 : 0;
            }
            if (lane < ncand && rank < kappa) {
                s_edges[rank] = pos;
                s_elab[rank] = lab;
            }
            if (lane == 0) s_ne = min(kappa, ncand);
        }
    } else if (wave == 0) {  // long token lists or degenerate weights: rounds over all tokens
        unsigned long long prev = ~0ull;
        int ne = 0;
        for (int r = 0; r < kappa; ++r) {
            unsigned long long best = 0ull;
            for (int j = lane; j < n; j += 64) {
                const int pos = tl[j];
                if (pos < p.n_sinks) continue;
                float w;
                if constexpr (NH == 1) {
                    w = p.logits[(size_t)g * p.t_cap + j];
                } else {
                    w = 0.f;
#pragma unroll
                    for (int h = 0; h < NH; ++h)
                        w += exp2f((p.logits[((size_t)g * NH + h) * p.t_cap + j] - M[h]) * kLog2e) * Linv[h];
                }
                const unsigned long long k = edge_key(w, pos);
                if (k < prev && k > best) best = k;
            }
            best = wave_max_u64(best);
            if (best == 0ull) break;
            const int pos = (int)(0xFFFFFFFFu - (uint32_t)best);
            if (lane == 0) {
                s_edges[r] = pos;
                s_elab[r] = p.label[(size_t)g * p.l_cap + pos];
            }
            prev = best;
            ++ne;
        }
        if (lane == 0) s_ne = ne;
    }
    // Meanwhile the other three waves combine the deferred gather's records
    // into the attention output.
    if constexpr (defer) {
        if (wave > 0) {
            float *o = p.out + ((size_t)gc.b * p.Hq + gc.qh0) * D;
            float *mlg = p.ml ? p.ml + (size_t)g * NH * 2 : nullptr;
            if (nact == 0) {
                combine_empty<D, NH, 192>(tid - 64, o, mlg);
            } else if constexpr (regs) {
                combine_out_regs<D, NH, 192, kPreChunks>(nact, s_comb, tid - 64, ov, o, mlg);
            } else {
                if (nact <= kCombineLds)
                    combine_out<D, NH, PS, false, 192>(PR, p.nchunk, nact, s_comb, tid - 64, o, mlg);
                else
                    combine_out_long<D, NH, PS, false, 192>(PR, p.nchunk, nact, tid - 64, o, mlg);
            }
        }
    }
    lds_barrier();
    const int ne = s_ne;
    const int P = s_P;
    const bool room = P < cap;
    CKV_TMARK(33);

    // Majority vote of the edges' labels, lowest id on ties: each edge counts
    // its label's votes; the largest (votes, ~label) wins.  No labelled edge:
    // the best-scoring community.
    if (wave == 0) {
        unsigned long long key = 0ull;
        if (lane < ne) {
            const int c = s_elab[lane];
            int k = 0;
            for (int r0 = 0; r0 < ne; r0 += 8) {  // ne <= 32 = CKV_MAX_KAPPA: reads stay inside s_elab
                int ll[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) ll[u] = s_elab[min(r0 + u, CKV_MAX_KAPPA - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u) k += (r0 + u < ne && ll[u] == c) ? 1 : 0;
            }
            if (c >= 0) key = ((unsigned long long)k << 32) | (0xFFFFFFFFu - (uint32_t)c);
        }
        key = wave_max_u64(key);
        const int a = key ? (int)(0xFFFFFFFFu - (uint32_t)key) : topc;
        if (lane < p.kappa) p.edges[(size_t)g * p.kappa + lane] = lane < ne ? s_edges[lane] : -1;  // kappa <= 32
        if (lane == 0) {
            p.assign[g] = a;
            s_a = a;
        }
    }
    lds_barrier();
    CKV_TMARK(34);

    // The graph of the group's first query head appends the new key and value
    // at position P (wave 3, idle in the update below; nothing in this kernel
    // reads the row).
    if (owner && room && wave == 3) {
        const int page = p.page_table[(size_t)gc.b * p.max_pages + (P >> p.ps_log2)];
        T *row = reinterpret_cast<T *>(p.kv) +
                 ((((size_t)page * p.Hkv + gc.kh) << p.ps_log2) | (size_t)(P & ((1 << p.ps_log2) - 1))) * (2 * D);
        for (int i = lane; i < 2 * D; i += 64) row[i] = i < D ? kn[i] : vn[i - D];
    }

    // Append to the winning community: label, tail entry, member count, the
    // float64 key sum and the float32 centroid column.
    const int a = s_a;
    const bool join = room && a >= 0 && tn < p.tail_cap;  // uniform
    int newsize = 0;
    float cv = 0.f;
    if (join && tid < D) {
        newsize = p.size[(size_t)g * p.c_cap + a] + 1;
        const size_t ci = ((size_t)g * p.c_cap + a) * D + tid;
        const double cs = p.csum[ci] + (double)to_f32(kn[tid]);
        p.csum[ci] = cs;
        if (p.vsum) p.vsum[ci] += (double)to_f32(vn[tid]);
        cv = (float)(cs / (double)newsize);
        p.cent[((size_t)g * p.c_cap + a) * D + tid] = cv;
    }
    // the screening copy of the column: scale = max |cent| / 127
    if (join) {
        const float m = wave_max_f(fabsf(cv));
        if (lane == 0) s_max[wave] = m;
    }
    if (tid == 0) {
        if (!room) {
            atomicOr(p.status, CKV_ST_CAPACITY);
        } else if (join) {
            p.label[(size_t)g * p.l_cap + P] = a;
            p.tail_pos[(size_t)g * p.tail_cap + tn] = P;
            p.tail_comm[(size_t)g * p.tail_cap + tn] = a;
            p.tail_len[g] = tn + 1;
        } else {
            if (a >= 0) atomicOr(p.status, CKV_ST_TAIL_FULL);
            p.label[(size_t)g * p.l_cap + P] = -1;
        }
    }
    CKV_TMARK(35);
    // Every thread has read the member count above: only now may it change.
    // The last block to count in advances every sequence with room by one
    // token; the next kernel sees it across the kernel boundary.
    __syncthreads();
    if (join) {
        const float scale = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])) / kScreenMax;
        if (tid < D) p.cq[cq_offset(g, tid, a, D, p.c_cap)] = screen_code(cv, scale);
        if (tid == 0) p.cscale[(size_t)g * p.c_cap + a] = scale;
    }
    if (tid == 0) {
        if (join) p.size[(size_t)g * p.c_cap + a] = newsize;
        if (last) {
            for (int bb = 0; bb < p.B; ++bb) {
                const int L0 = few ? s_len[bb] : p.seq_len[bb];
                if (L0 < cap) p.seq_len[bb] = L0 + 1;
            }
            reset_counter(p.ctr);
        }
    }
    CKV_TMARK(36);
}

hipError_t launch_assign(const ckv_kv *kv, const ckv_index *idx, const int32_t *tok_list,
                         const int32_t *tok_n, const float *logits, float *ml, int t_cap,
                         const int32_t *top, int kappa, const void *k_new, const void *v_new,
                         int32_t *edges, int32_t *assign, float *out, const float *part, int32_t *ctr,
                         hipStream_t s) {
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
    p.G = idx->n_graphs;  // arrivals of every window of the step
    const Window w = window_of(idx);
    p.g0 = w.first;
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
    p.cq = idx->cq;
    p.cscale = idx->cscale;
    p.status = idx->status;
    p.tok_list = tok_list;
    p.tok_n = tok_n;
    p.logits = logits;
    p.ml = ml;
    p.out = out;
    p.part = part;
    p.nchunk = gather_slots(idx, t_cap);
    p.cent_n = idx->cent_budget > 0 ? idx->cent_n : nullptr;
    p.vsum = idx->cent_budget > 0 ? idx->vsum : nullptr;
    p.top = top;
    p.k_new = k_new;
    p.v_new = v_new;
    p.edges = edges;
    p.assign = assign;
    p.ctr = ctr;
    const int nh = heads_per_graph(kv, idx);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    const dim3 grid(w.count), block(256);
    const int mode = !out ? kAssignComplete : (nh <= 4 && p.nchunk <= kPreChunks) ? kAssignDeferRegs : kAssignDefer;
#define CKV_AS_M(TT, DD, NN, MM)                                                  \
    if (kv->head_dim == DD && nh == NN && mode == MM) {                          \
        CKV_LAUNCH((assign_kernel<TT, DD, NN, MM>), grid, block, s, p);          \
        return hipGetLastError();                                                \
    }
#define CKV_AS(TT, DD, NN)                        \
    CKV_AS_M(TT, DD, NN, kAssignComplete)         \
    CKV_AS_M(TT, DD, NN, kAssignDefer)            \
    CKV_AS_M(TT, DD, NN, (NN <= 4 ? kAssignDeferRegs : kAssignDefer))
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
#undef CKV_AS_M
    return hipErrorInvalidValue;
}

}  // namespace ckv
