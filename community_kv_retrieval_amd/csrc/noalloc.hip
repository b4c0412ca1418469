// ckv_gather_attend_noalloc: the gather of ckv_gather_attend (complete mode)
// for callers that cannot allocate device memory, with its split-K partial
// records and arrival counters in a static device array of this library
// instead of a caller workspace.
//
// The array is one per GPU (each device that loads the code object holds its
// own copy, at its own address).  Host code never passes the array's name to a
// kernel: the name is a host-side stand-in.  The device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and kept.
// Every call on a device shares that device's array, so calls that overlap on
// one GPU (different streams, or different host threads) race; calls ordered
// on one stream do not.  Each call clears the counters it uses with a fill
// kernel before the gather (no hipMemsetAsync, so a captured call replays
// correctly).
#include <mutex>

#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {
namespace {

static __device__ __align__(256) unsigned char scratch[CKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

// Bytes of scratch a gather of this shape uses: the arrival counters of every
// graph, then one partial record per graph, head and record slot (as in the
// workspace).
size_t noalloc_gather_bytes(const ckv_kv *kv, const ckv_index *idx, int t_cap) {
    const size_t G = (size_t)idx->n_graphs;
    const size_t ctr = align256(4 * G);
    const size_t part = align256(4 * G * heads_per_graph(kv, idx) * (size_t)gather_slots(idx, t_cap) *
                                 (size_t)part_stride(kv->head_dim));
    return ctr + part;
}

hipError_t launch_gather_noalloc(const ckv_kv *kv, const ckv_index *idx, const void *q, const int32_t *tok_list,
                                 const int32_t *tok_n, int t_cap, float sm_scale, float *out, float *logits,
                                 float *ml, hipStream_t s) {
    void *base = nullptr;
    hipError_t e = scratch_address(&base);
    if (e != hipSuccess) return e;
    int32_t *ctr = static_cast<int32_t *>(base);
    float *part = reinterpret_cast<float *>(static_cast<unsigned char *>(base) + align256(4 * (size_t)idx->n_graphs));
    hipLaunchKernelGGL(zero_i32_kernel, dim3(ceil_div(idx->n_graphs, 256)), dim3(256), 0, s, ctr, idx->n_graphs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gather(kv, idx, q, tok_list, tok_n, t_cap, sm_scale, out, logits, ml, part, ctr, s);
}

}  // namespace ckv
