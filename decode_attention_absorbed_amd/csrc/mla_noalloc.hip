// mla_decode_attn_noalloc: the decode step with its scratch memory in a
// buffer the library itself holds on each device, for callers that cannot
// allocate (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc).  The kernels are mla_decode_attn's; only where the
// scratch comes from differs.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdio.h>

#include "mla_internal.hpp"

namespace {

// The scratch buffer: one copy per device, held until the process ends.
// In host code `scratch` names a host-side stand-in, never the device
// memory; the device address comes from hipGetSymbolAddress below.
__device__ __attribute__((aligned(256))) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once
// per device with that device current.
hipError_t scratch_address(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" int mla_decode_attn_noalloc(mla_decode_params_t* p, void* stream) {
    if (!p) return mla::set_error(MLA_ERR_INVALID_ARG, "mla_decode_attn_noalloc: null params");
    // Sizes the planner rejects get mla_decode_attn's own message below.
    const size_t need = mla_decode_workspace_size(p->B, p->H, p->K, p->dtype_act, p->dtype_w, p->num_cus,
                                                  p->num_splits);
    if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) {
        char msg[200];
        snprintf(msg, sizeof msg,
                 "mla_decode_attn_noalloc: these sizes need %zu bytes of scratch, more than the %zu-byte buffer",
                 need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
        return mla::set_error(MLA_ERR_WORKSPACE, msg);
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return mla::set_error(MLA_ERR_HIP, "mla_decode_attn_noalloc: cannot query the current device");
    void* ptr = nullptr;
    const hipError_t e = scratch_address(dev, &ptr);
    if (e != hipSuccess) {
        char msg[200];
        snprintf(msg, sizeof msg, "mla_decode_attn_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
        return mla::set_error(MLA_ERR_HIP, msg);
    }
    mla_decode_params_t q = *p;
    q.workspace = ptr;
    q.workspace_size = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
    const int rc = mla_decode_attn(&q, stream);
    p->validate_status = q.validate_status;
    return rc;
}
