// Paged K/V writes and the community index build.
//
// The build turns a given partition (the CommunityKV page, Figure 1 panel
// (2): communities of the prefill token graph, each with a centroid) into the
// decode-time index: member counts, a community-ordered CSR of positions, the
// per-position labels, and per community the exact float64 sum of the members'
// keys with its float32 mean (the centroid), one row per community, and the
// int8 screening copy of that row for the scoring kernel.  Steps: clear,
// count (atomic increments), one block scan per graph, scatter (atomic
// cursors), then one block per community that sorts its
// members by position (so the CSR does not depend on atomic order: a rank
// sort in LDS, or for communities of more than 2048 members an ordered pass
// over the labels) and sums their keys in that order.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

template <typename T>
__global__ __launch_bounds__(256) void kv_write_kernel(T *kv, const int32_t *ptab, int Hkv,
                                                       int ps_log2, int D, int kh, int pos0, int n,
                                                       const T *k, const T *v) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t per = 2 * (size_t)D;
    if (i >= (size_t)n * per) return;
    const int t = (int)(i / per), r = (int)(i - (size_t)t * per);
    const int pos = pos0 + t;
    const int page = ptab[pos >> ps_log2];
    const size_t row = (((size_t)page * Hkv + kh) << ps_log2) | (size_t)(pos & ((1 << ps_log2) - 1));
    kv[row * per + r] = r < D ? k[(size_t)t * D + r] : v[(size_t)t * D + r - D];
}

hipError_t launch_kv_write(const ckv_kv *kv, int b, int kh, int pos0, int n, const void *k,
                           const void *v, hipStream_t s) {
    const size_t total = (size_t)n * 2 * kv->head_dim;
    const dim3 grid((unsigned)((total + 255) / 256));
    const int ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    const int32_t *ptab = kv->page_table + (size_t)b * kv->max_pages;
    if (kv->dtype == CKV_DTYPE_BF16)
        hipLaunchKernelGGL(kv_write_kernel<bf16_t>, grid, dim3(256), 0, s, (bf16_t *)kv->kv, ptab,
                           kv->n_kv_heads, ps_log2, kv->head_dim, kh, pos0, n, (const bf16_t *)k,
                           (const bf16_t *)v);
    else
        hipLaunchKernelGGL(kv_write_kernel<float>, grid, dim3(256), 0, s, (float *)kv->kv, ptab,
                           kv->n_kv_heads, ps_log2, kv->head_dim, kh, pos0, n, (const float *)k,
                           (const float *)v);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

static hipError_t fill_u32(void *p, size_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                       (uint32_t *)p, n, v);
    return hipGetLastError();
}

struct BuildParams {
    const void *kv;
    const int32_t *page_table;
    const int32_t *seq_len;
    const int32_t *labels_in;
    int Hq, Hkv, ps_log2, max_pages;
    int mode, c_cap, l_cap, n_sinks;
    int32_t *n_comm;
    int32_t *size;
    int32_t *offs;
    int32_t *toks;
    int32_t *label;
    double *csum;
    double *vsum;  // centroid budget: value sums (else null)
    float *cent;
    int8_t *cq;
    float *cscale;
    int32_t *status;
    int32_t *cursor;
};

__global__ __launch_bounds__(256) void build_count_kernel(BuildParams p) {
    const int g = blockIdx.y;
    const int pos = blockIdx.x * 256 + threadIdx.x;
    if (pos >= p.l_cap) return;
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int L = p.seq_len[gc.b];
    int lab = (pos < L && pos >= p.n_sinks) ? p.labels_in[(size_t)g * p.l_cap + pos] : -1;
    if (lab >= min(p.n_comm[g], p.c_cap)) {
        atomicOr(p.status, CKV_ST_BAD_LABEL);
        lab = -1;
    }
    if (lab < -1) lab = -1;
    p.label[(size_t)g * p.l_cap + pos] = lab;
    if (lab >= 0) atomicAdd(&p.size[(size_t)g * p.c_cap + lab], 1);
}

template <int EPT>
__global__ __launch_bounds__(1024) void build_scan_kernel(BuildParams p) {
    __shared__ int scratch[1024 / 64 + 1];
    const int g = blockIdx.x, tid = threadIdx.x;
    const int32_t *sz = p.size + (size_t)g * p.c_cap;
    int v[EPT], loc = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid * EPT + j;
        v[j] = c < p.c_cap ? sz[c] : 0;
        loc += v[j];
    }
    int total;
    int run = block_exclusive_scan<1024>(loc, scratch, &total);
    int32_t *offs = p.offs + (size_t)g * offs_stride(p.c_cap);
    int32_t *cur = p.cursor + (size_t)g * p.c_cap;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int c = tid * EPT + j;
        if (c < p.c_cap) {
            offs[c] = run;
            cur[c] = run;
        }
        run += v[j];
    }
    if (tid == 0) offs[p.c_cap] = total;
}

__global__ __launch_bounds__(256) void build_scatter_kernel(BuildParams p) {
    const int g = blockIdx.y;
    const int pos = blockIdx.x * 256 + threadIdx.x;
    if (pos >= p.l_cap) return;
    const int lab = p.label[(size_t)g * p.l_cap + pos];
    if (lab < 0) return;
    const int slot = atomicAdd(&p.cursor[(size_t)g * p.c_cap + lab], 1);
    p.toks[(size_t)g * p.l_cap + slot] = pos;
}

constexpr int kSortMax = 2048;

template <typename T, int D>
__global__ __launch_bounds__(256) void build_finish_kernel(BuildParams p) {
    __shared__ int buf[kSortMax];
    const int g = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    if (c >= min(p.n_comm[g], p.c_cap)) return;
    const int32_t *offs = p.offs + (size_t)g * offs_stride(p.c_cap);
    const int o = offs[c], s = offs[c + 1] - o;
    if (s <= 0) return;
    int32_t *mem = p.toks + (size_t)g * p.l_cap + o;
    if (s <= kSortMax) {
        for (int i = tid; i < s; i += 256) buf[i] = mem[i];
        __syncthreads();
        for (int i = tid; i < s; i += 256) {
            const int x = buf[i];
            int r = 0;
            for (int j = 0; j < s; ++j) r += buf[j] < x;
            mem[r] = x;
        }
    } else {
        // Large community: its members are exactly the positions labelled c,
        // so one ordered pass over the graph's labels lists them ascending.
        // Thread t counts its run of positions, a block scan gives each run
        // its first slot, and the run writes its members in order.
        const int32_t *lab = p.label + (size_t)g * p.l_cap;
        const int per = (p.l_cap + 255) / 256;
        const int q0 = min(tid * per, p.l_cap), q1 = min(q0 + per, p.l_cap);
        int cnt = 0;
        for (int q = q0; q < q1; ++q) cnt += lab[q] == c ? 1 : 0;
        int total;
        int k = block_exclusive_scan<256>(cnt, buf, &total);
        for (int q = q0; q < q1; ++q)
            if (lab[q] == c) mem[k++] = q;
    }
    __syncthreads();
    __threadfence_block();
    const GraphCoords gc = graph_coords(g, p.mode, p.Hq, p.Hkv);
    const int32_t *ptab = p.page_table + (size_t)gc.b * p.max_pages;
    const T *kvb = reinterpret_cast<const T *>(p.kv);
    const int smask = (1 << p.ps_log2) - 1;
    static_assert(2 * D <= 256, "one thread per dimension of the key sum and of the value sum");
    __shared__ float s_max[4];
    float cv = 0.f;
    if (tid < D) {
        double acc = 0.0;
        for (int i = 0; i < s; ++i) {
            const int pos = mem[i];
            const int page = ptab[pos >> p.ps_log2];
            const size_t row = (((size_t)page * p.Hkv + gc.kh) << p.ps_log2) | (size_t)(pos & smask);
            acc += (double)to_f32(kvb[row * 2 * D + tid]);
        }
        p.csum[((size_t)g * p.c_cap + c) * D + tid] = acc;
        cv = (float)(acc / (double)s);
        p.cent[((size_t)g * p.c_cap + c) * D + tid] = cv;
    } else if (p.vsum && tid < 2 * D) {  // value sums, in the same member order
        const int e = tid - D;
        double acc = 0.0;
        for (int i = 0; i < s; ++i) {
            const int pos = mem[i];
            const int page = ptab[pos >> p.ps_log2];
            const size_t row = (((size_t)page * p.Hkv + gc.kh) << p.ps_log2) | (size_t)(pos & smask);
            acc += (double)to_f32(kvb[row * 2 * D + D + e]);
        }
        p.vsum[((size_t)g * p.c_cap + c) * D + e] = acc;
    }
    // screening copy of the column: scale = max |cent| / 127
    const float m = wave_max_f(fabsf(cv));
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    const float scale = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3])) / kScreenMax;
    if (tid < D) p.cq[cq_offset(g, tid, c, D, p.c_cap)] = screen_code(cv, scale);
    if (tid == 0) p.cscale[(size_t)g * p.c_cap + c] = scale;
}

hipError_t launch_index_build(const ckv_kv *kv, const ckv_index *idx, const int32_t *labels_in,
                              int32_t *cursor, hipStream_t s) {
    const size_t G = (size_t)idx->n_graphs, C = (size_t)idx->c_cap, D = (size_t)kv->head_dim;
    hipError_t e;
    if ((e = fill_u32(idx->size, G * C, 0u, s)) != hipSuccess) return e;
    if ((e = fill_u32(idx->csum, G * C * D * 2, 0u, s)) != hipSuccess) return e;
    if (idx->cent_budget > 0 && (e = fill_u32(idx->vsum, G * C * D * 2, 0u, s)) != hipSuccess) return e;
    if ((e = fill_u32(idx->cent, G * C * D, 0u, s)) != hipSuccess) return e;
    if ((e = fill_u32(idx->cq, G * C * D / 4, 0u, s)) != hipSuccess) return e;  // C % 256 == 0
    if ((e = fill_u32(idx->cscale, G * C, 0u, s)) != hipSuccess) return e;
    if ((e = fill_u32(idx->tail_len, G, 0u, s)) != hipSuccess) return e;
    if ((e = fill_u32(idx->status, 1, 0u, s)) != hipSuccess) return e;

    BuildParams p{};
    p.kv = kv->kv;
    p.page_table = kv->page_table;
    p.seq_len = kv->seq_len;
    p.labels_in = labels_in;
    p.Hq = kv->n_q_heads;
    p.Hkv = kv->n_kv_heads;
    p.ps_log2 = __builtin_ctz((unsigned)kv->page_size);
    p.max_pages = kv->max_pages;
    p.mode = idx->mode;
    p.c_cap = idx->c_cap;
    p.l_cap = idx->l_cap;
    p.n_sinks = idx->n_sinks;
    p.n_comm = idx->n_comm;
    p.size = idx->size;
    p.offs = idx->offs;
    p.toks = idx->toks;
    p.label = idx->label;
    p.csum = idx->csum;
    p.vsum = idx->cent_budget > 0 ? idx->vsum : nullptr;
    p.cq = idx->cq;
    p.cscale = idx->cscale;
    p.cent = idx->cent;
    p.status = idx->status;
    p.cursor = cursor;

    const dim3 gpos(ceil_div(idx->l_cap, 256), (unsigned)G);
    hipLaunchKernelGGL(build_count_kernel, gpos, dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ept = ceil_div(idx->c_cap, 1024);
    if (ept <= 1) hipLaunchKernelGGL(build_scan_kernel<1>, dim3((unsigned)G), dim3(1024), 0, s, p);
    else if (ept <= 2) hipLaunchKernelGGL(build_scan_kernel<2>, dim3((unsigned)G), dim3(1024), 0, s, p);
    else if (ept <= 4) hipLaunchKernelGGL(build_scan_kernel<4>, dim3((unsigned)G), dim3(1024), 0, s, p);
    else if (ept <= 8) hipLaunchKernelGGL(build_scan_kernel<8>, dim3((unsigned)G), dim3(1024), 0, s, p);
    else hipLaunchKernelGGL(build_scan_kernel<16>, dim3((unsigned)G), dim3(1024), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(build_scatter_kernel, gpos, dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 gcomm((unsigned)C, (unsigned)G);
    const bool bf = kv->dtype == CKV_DTYPE_BF16;
    if (kv->head_dim == 128) {
        if (bf) hipLaunchKernelGGL((build_finish_kernel<bf16_t, 128>), gcomm, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((build_finish_kernel<float, 128>), gcomm, dim3(256), 0, s, p);
    } else {
        if (bf) hipLaunchKernelGGL((build_finish_kernel<bf16_t, 64>), gcomm, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((build_finish_kernel<float, 64>), gcomm, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace ckv
