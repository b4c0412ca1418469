// Attention-mass recall (the CommunityKV page, Figure 3): the share of a
// head's dense softmax mass that the tokens attended by the sparse step
// carry.  Both softmax states are (max m, sum l = sum_j exp(z_j - m)) over
// their token sets, so the attended mass over the total mass is
//   exp(m_T - m_all) * l_T / l_all,
// evaluated here in float64 as exp((m_T - m_all) + log l_T - log l_all).
#include <hip/hip_runtime.h>

#include "ckv_internal.h"

namespace ckv {
namespace {

__global__ void recall_kernel(const float *__restrict__ ml, const float *__restrict__ dense_ml,
                              float *__restrict__ recall, int G, int hpg, int n_q_heads, int n_kv_heads,
                              int per_head) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= G * hpg) return;
    const int g = i / hpg, h = i - g * hpg;
    int b, qh;
    if (per_head) {
        b = g / n_q_heads;
        qh = g - b * n_q_heads;
    } else {
        b = g / n_kv_heads;
        qh = (g - b * n_kv_heads) * hpg + h;
    }
    const float mt = ml[2 * i], lt = ml[2 * i + 1];
    const size_t d = 2 * ((size_t)b * n_q_heads + qh);
    const float md = dense_ml[d], ld = dense_ml[d + 1];
    float r = 0.f;  // nothing attended: no mass
    if (lt > 0.f && ld > 0.f)
        r = (float)exp(((double)mt - (double)md) + log((double)lt) - log((double)ld));
    recall[i] = r;
}

}  // namespace

hipError_t launch_recall(const ckv_kv *kv, const ckv_index *idx, const float *ml, const float *dense_ml,
                         float *recall, hipStream_t s) {
    const int hpg = heads_per_graph(kv, idx);
    const int n = idx->n_graphs * hpg;
    CKV_LAUNCH(recall_kernel, dim3(ceil_div(n, 256)), dim3(256), s, ml, dense_ml, recall, idx->n_graphs, hpg,
               kv->n_q_heads, kv->n_kv_heads, idx->mode == CKV_MODE_PER_HEAD ? 1 : 0);
    return hipGetLastError();
}

}  // namespace ckv
