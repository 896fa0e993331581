// sa_sparse_attn_noalloc (include/sa.h): sparse_attn for callers that cannot allocate device
// memory. The workspace (split partials, dequantised rows) lives in a static device array of
// the library instead of a caller buffer; everything else is sa_sparse_attn's own path (same
// plan, same kernels).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sa.h"
#include "sa_internal.hpp"

#define SA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;

// One copy per GPU, held until the process ends. In host code `scratch` is only a stand-in
// for the symbol: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of the current device's copy of `scratch`, looked up on the first call
// on that device (with it current) and kept.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SA_OK;
}

}  // namespace

SA_EXPORT int sa_sparse_attn_noalloc(const sa_attn_args* a, void* stream) {
    // the size check needs no HIP call beyond the compute-unit count the plan uses
    size_t need = 0;
    int rc = sa_sparse_attn_workspace(a, &need);
    if (rc != SA_OK) return rc;
    if (need > kScratchBytes) return SA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        rc = scratch_address(&ws);
        if (rc != SA_OK) return rc;
    }
    sa::KParams p;
    sa::Plan pl;
    rc = sa::prepare_sparse_attn(a, ws, kScratchBytes, p, pl);
    if (rc != SA_OK) return rc;
    const hipError_t e = sa::run_sparse_attn(a, p, pl, (hipStream_t)stream);
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}
