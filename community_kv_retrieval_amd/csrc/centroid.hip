// Centroid terms of the centroid budget (the CommunityKV page, Table 6,
// "Centroid Budget").  Each community that the centroid selection chose
// enters the attention as one softmax term standing for its n members: key
// mu = the stored float32 centroid row (float32(csum / n)); value
// float32(vsum / n), the members' mean value; logit sm_scale * q . mu + ln n
// (the mass of n tokens whose key is the centroid).
//
// One 256-thread block per graph and group of kCentPerRecord (16) terms, laid
// out like a gather block: 16-lane rows, row r taking the group's term r;
// lane l16 of a row holds dimensions [l16 E, l16 E + E) of mu (from the
// centroid row) and of the value (E = D / 16; the float64 value sum divided
// once).  The four rows
// of a wave merge their softmax states with lane shuffles, the four waves in
// a fixed order through LDS.  Each block's result is one more partial record
// of the gather: group j of a graph goes to the slot ceil(tok_n / 256) + j,
// right after the graph's spans, and the gather's combine (or the assign
// kernel's, for a deferred gather) takes those records after the spans'.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

struct CentParams {
    const void *q;
    const float *cent;
    const double *vsum;
    const int32_t *size;
    const int32_t *cent_sel;
    const int32_t *cent_n;
    const int32_t *tok_n;
    float *part;
    float sm_scale;
    int mode, Hq, Hkv, c_cap, N, nslots, g0, count;
};

template <typename T, int D, int NH>
__global__ __launch_bounds__(256) void centroid_attend_kernel(CentParams p) {
    constexpr int E = D / 16;
    constexpr int PS = part_stride(D);
    constexpr int kRows = 16;  // 16-lane rows per block
    __shared__ float s_q[NH][D];
    __shared__ float s_wm[4][NH], s_wl[4][NH];
    __shared__ float s_wacc[4][NH][D];
    // Group-major order: group j of every graph of the window before group j + 1.
    const int grp = blockIdx.x / p.count, g = p.g0 + (blockIdx.x - grp * p.count);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid >> 4, l16 = tid & 15;
    const int nce = p.cent_n[g];
    if (grp * kCentPerRecord >= nce) return;  // uniform: no terms in this group, no record
    const int n = p.tok_n[g];
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const T *qp = reinterpret_cast<const T *>(p.q) + ((size_t)gc.b * p.Hq + gc.qh0) * D;
    for (int i = tid; i < NH * D; i += 256) s_q[i / D][i % D] = to_f32(qp[i]);
    __syncthreads();
    float qr[NH][E];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) qr[h][e] = s_q[h][l16 * E + e];

    float m[NH], l[NH], acc[NH][E];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }
    static_assert(kRows == kCentPerRecord, "one term per row");
    const int term = grp * kCentPerRecord + row;
    if (term < nce) {
        const int c = p.cent_sel[(size_t)g * p.N + term];
        const int cnt = p.size[(size_t)g * p.c_cap + c];
        const size_t off = ((size_t)g * p.c_cap + c) * D + l16 * E;
        float mu[E];
        double vd[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            mu[e] = p.cent[off + e];
            vd[e] = p.vsum[off + e];
        }
        const double dn = (double)cnt;
        const float lnn = logf((float)cnt);
        float nu[E];
#pragma unroll
        for (int e = 0; e < E; ++e) nu[e] = (float)(vd[e] / dn);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) d = fmaf(qr[h][e], mu[e], d);
            d = row16_sum(d);
            const float z = fmaf(d, p.sm_scale, lnn);
            const float mn = fmaxf(m[h], z);
            const float sc = (m[h] == kNegInf) ? 0.f : exp2f((m[h] - mn) * kLog2e);
            const float pz = exp2f((z - mn) * kLog2e);
            l[h] = l[h] * sc + pz;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pz, nu[e], acc[h][e] * sc);
            m[h] = mn;
        }
    }
    // Merge the wave's four rows (lanes l16, l16 + 16, l16 + 32, l16 + 48).
#pragma unroll
    for (int h = 0; h < NH; ++h) {
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
            const float mo = shfl_xor_f(m[h], msk), lo = shfl_xor_f(l[h], msk);
            float M, s1, s2;
            softmax_scales(m[h], mo, M, s1, s2);
            l[h] = l[h] * s1 + lo * s2;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float ao = shfl_xor_f(acc[h][e], msk);
                acc[h][e] = acc[h][e] * s1 + ao * s2;
            }
            m[h] = M;
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if (lane == 0) {
                s_wm[wave][h] = m[h];
                s_wl[wave][h] = l[h];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) s_wacc[wave][h][l16 * E + e] = acc[h][e];
        }
    }
    __syncthreads();
    // The four waves in a fixed order; the record goes to slot ceil(n / 256) +
    // grp, after the graph's spans (n <= t_cap and grp < cent_records(N), so
    // the slot is below nslots).
    const int slot = (n > 0 ? (n + kGatherTokens - 1) / kGatherTokens : 0) + grp;
    float *P = p.part + (size_t)g * NH * p.nslots * PS;
    for (int i = tid; i < NH * D; i += 256) {
        const int h = i / D, d = i - (i / D) * D;
        float M = s_wm[0][h];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, s_wm[w][h]);
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float s = (s_wm[w][h] == kNegInf) ? 0.f : exp2f((s_wm[w][h] - M) * kLog2e);
            o += s_wacc[w][h][d] * s;
            L += s_wl[w][h] * s;
        }
        float *dst = P + ((size_t)h * p.nslots + slot) * PS;
        dst[d] = o;
        if (d == 0) {
            dst[D] = M;
            dst[D + 1] = L;
        }
    }
}

hipError_t launch_centroid_attend(const ckv_kv *kv, const ckv_index *idx, const void *q, const int32_t *tok_n,
                                  float sm_scale, float *part, int nslots, hipStream_t s) {
    CentParams p{};
    p.q = q;
    p.cent = idx->cent;
    p.vsum = idx->vsum;
    p.size = idx->size;
    p.cent_sel = idx->cent_sel;
    p.cent_n = idx->cent_n;
    p.tok_n = tok_n;
    p.part = part;
    p.sm_scale = sm_scale;
    p.mode = idx->mode;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.c_cap = idx->c_cap;
    p.N = idx->cent_budget;
    p.nslots = nslots;
    const Window w = window_of(idx);
    p.g0 = w.first;
    p.count = w.count;
    const int nh = heads_per_graph(kv, idx);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    const dim3 grid(w.count * cent_records(idx->cent_budget)), block(256);
#define CKV_CENT(TT, DD, NN)                                                          \
    if (kv->head_dim == DD && nh == NN) {                                             \
        hipLaunchKernelGGL((centroid_attend_kernel<TT, DD, NN>), grid, block, 0, s, p); \
        return hipGetLastError();                                                     \
    }
#define CKV_CENT_T(TT)                                                                \
    CKV_CENT(TT, 64, 1) CKV_CENT(TT, 64, 2) CKV_CENT(TT, 64, 4) CKV_CENT(TT, 64, 8)   \
    CKV_CENT(TT, 128, 1) CKV_CENT(TT, 128, 2) CKV_CENT(TT, 128, 4) CKV_CENT(TT, 128, 8)
    if (bf) {
        CKV_CENT_T(bf16_t)
    } else {
        CKV_CENT_T(float)
    }
#undef CKV_CENT_T
#undef CKV_CENT
    return hipErrorInvalidValue;
}

}  // namespace ckv
