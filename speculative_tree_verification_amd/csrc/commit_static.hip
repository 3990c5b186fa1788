// commit_static.hip -- tree_ssd_commit_layers_static: the multi-layer commit
// for callers that cannot allocate device memory. tree_ssd_commit_layers
// reads its layer table from a device array the caller provides; this entry
// point takes the table in host memory and stages it into a fixed array of
// device memory owned by the library (one copy per GPU), then runs the same
// commit kernel on it. No device memory is allocated or freed by the call.
//
// The table reaches the GPU as kernel arguments of a staging kernel (64
// layers per launch), so the caller's host array may be reused as soon as
// the call returns; nothing is read from it later.
#include <mutex>

#include "launch.hpp"
#include "tree_ssd.h"

namespace {

constexpr int kStaticMaxLayers = TSV_STATIC_MAX_LAYERS;
constexpr int kStageChunk = 64;  // layers per staging launch: 64 x 40 B of kernel arguments
constexpr int kMaxDevices = 64;

struct LayerChunk {
    tsv_commit_layer l[kStageChunk];
};

__global__ void __launch_bounds__(kStageChunk)
stage_layers_kernel(LayerChunk c, tsv_commit_layer* __restrict__ dst, int count) {
    const int i = threadIdx.x;
    if (i < count) dst[i] = c.l[i];
}

}  // namespace

// The layer table of tree_ssd_commit_layers_static. Host code never uses this
// name as an address: it is resolved per device with hipGetSymbolAddress.
static __device__ __align__(256) tsv_commit_layer scratch[kStaticMaxLayers];

namespace {

std::mutex g_scratch_mu;
tsv_commit_layer* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call made with that device current.
hipError_t scratch_table(tsv_commit_layer** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<tsv_commit_layer*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" tsv_status tree_ssd_commit_layers_static(const tsv_shape* s, int32_t n_layers,
                                                    const tsv_commit_layer* layers_host,
                                                    const int32_t* parent, const int32_t* accepted,
                                                    const int32_t* accepted_len, int32_t max_path_len,
                                                    int32_t* tree_status, void* stream) {
    bool nothing = false;
    tsv_status st = tsv::check_commit_layers(s, n_layers, parent, accepted, accepted_len, max_path_len, &nothing);
    if (st != TSV_OK || nothing) return st;
    if (n_layers > kStaticMaxLayers) return TSV_E_UNSUPPORTED;
    if (!layers_host) return TSV_E_NULL;
    tsv_commit_layer* table = nullptr;
    if (scratch_table(&table) != hipSuccess) return TSV_E_LAUNCH;
    hipStream_t hs = (hipStream_t)stream;
    for (int first = 0; first < n_layers; first += kStageChunk) {
        const int count = n_layers - first < kStageChunk ? n_layers - first : kStageChunk;
        LayerChunk c{};
        for (int i = 0; i < count; ++i) c.l[i] = layers_host[first + i];
        hipLaunchKernelGGL(stage_layers_kernel, dim3(1), dim3(kStageChunk), 0, hs, c, table + first, count);
        if (hipGetLastError() != hipSuccess) return TSV_E_LAUNCH;
    }
    hipError_t e = tsv::launch_commit(tsv::layers_args(s, n_layers, table, parent, accepted, accepted_len,
                                                       max_path_len, tree_status),
                                      s->in_dtype == TSV_BF16, hs);
    return e == hipSuccess ? TSV_OK : TSV_E_LAUNCH;
}
