// noalloc.hip -- piattn_fwd_noalloc: the prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The workspace piattn_fwd takes from the
// caller comes instead from `scratch`, a file-scope device array of
// PIATTN_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends.
//
// On the host the array's name is only a stand-in for its device address, so
// the address is looked up once per device (with that device current) by
// hipGetSymbolAddress and cached; kernels receive the cached pointer as their
// workspace argument, exactly as they receive a caller's workspace.
#include <mutex>

#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "api_internal.hpp"
#include "piattn.h"

namespace {

__device__ __align__(256) unsigned char scratch[PIATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on first use).
int scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return api_fail(PIATTN_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return api_fail(PIATTN_EUNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                        kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return api_fail(PIATTN_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                            hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PIATTN_OK;
}

}  // namespace

extern "C" int piattn_fwd_noalloc(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q,
                                  const void* k, const void* v, const float* gate_logits, void* out,
                                  float* lse_out, const int64_t strides[5][3], const int32_t* cu_seqlens,
                                  const piattn_pattern* pattern, void* stream) {
    int rc = api_check_fwd(dtype, B, H, n, d, q, k, v, gate_logits, out, lse_out, strides, cu_seqlens, pattern);
    if (rc) return rc;
    const size_t need = piattn_fwd_workspace_bytes(dtype, B, H, n, d, pattern);
    if (need > (size_t)PIATTN_NOALLOC_SCRATCH_BYTES)
        return api_fail(PIATTN_EWORKSPACE,
                        "this call needs %zu bytes of scratch; the library-held array has %zu "
                        "(PIATTN_NOALLOC_SCRATCH_BYTES): use piattn_fwd with a workspace",
                        need, (size_t)PIATTN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return piattn_fwd(dtype, B, H, n, d, q, k, v, gate_logits, out, lse_out, strides, cu_seqlens, pattern, ws,
                      (size_t)PIATTN_NOALLOC_SCRATCH_BYTES, stream);
}
