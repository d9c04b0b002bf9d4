// fsl_attn_fwd_noalloc: the whole forward with its workspace in a device array
// that the library itself holds, for callers that cannot allocate (code under
// stream capture, tight serving loops, hosts that forbid allocation calls).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, at its own address, from the first call on that device
// until the process ends. Its host-side name is only a stand-in for the symbol,
// so the device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and that address is what the kernels receive. Nothing
// here calls hipMalloc or hipFree. The forward writes every workspace word it
// later reads, so the array needs no clearing between calls; calls that overlap
// on one GPU share the array and race.
#include <mutex>

#include "fsl_internal.h"

static_assert(FSL_NOALLOC_WORKSPACE_MAX % 256 == 0, "whole 256-byte units");
static __device__ __align__(256) uint8_t scratch[FSL_NOALLOC_WORKSPACE_MAX];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// the current device's copy of the array (looked up on the first call per device)
int scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FSL_E_HIP;
    if (dev >= kMaxDevices) return FSL_E_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FSL_E_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return FSL_OK;
}

}  // namespace

extern "C" int fsl_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, const fsl_params *p,
                                    int32_t *sel_out, float *o_win_out, float *o_long_out, hipStream_t stream) {
    const int rc = fsl_check_params(p);
    if (rc != FSL_OK) return rc;
    if (fsl_workspace_bytes(p) > (size_t)FSL_NOALLOC_WORKSPACE_MAX) return FSL_E_WORKSPACE;
    if (!q || !k || !v || !out) return FSL_E_INVAL;
    void *ws = nullptr;
    const int src = scratch_for_current_device(&ws);
    if (src != FSL_OK) return src;
    return fsl_attn_fwd(q, k, v, out, p, ws, (size_t)FSL_NOALLOC_WORKSPACE_MAX, sel_out, o_win_out, o_long_out,
                        stream);
}
