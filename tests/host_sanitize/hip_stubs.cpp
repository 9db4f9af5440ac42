// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// libmla_decode's host code makes, so that its argument checks, split plan
// and workspace layout can run under AddressSanitizer and UBSan on the CPU.
// The launch stand-ins write every byte of each workspace region the plan
// hands the kernels, so a region that runs past the workspace the caller
// sized with mla_decode_workspace_size is reported as a heap overflow.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../decode_attention_absorbed_amd/csrc/mla_internal.hpp"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t) { memset(p, v, n); return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) {
    memcpy(d, s, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

namespace mla {

static size_t act_bytes(const Plan& pl) { return pl.bf16_path ? 2 : 4; }

hipError_t launch_rope_freqs(const mla_rope_cfg_t&, float*, hipStream_t) { ++g_launches; return hipSuccess; }

hipError_t launch_prep(const mla_decode_params_t& p, const Plan& pl, const Work& w, bool, hipStream_t) {
    ++g_launches;
    memset(w.qt, 0, (size_t)p.B * p.H * 576 * act_bytes(pl));
    if (pl.bf16_path) memset(w.qlo, 0, (size_t)p.B * p.H * 64 * 2);
    memset(w.list, 0, (size_t)p.B * p.K * 4);
    memset(w.counts, 0, (size_t)p.B * 4);
    memset(w.status, 0, 4);
    return hipSuccess;
}

hipError_t launch_attn(const mla_decode_params_t& p, const Plan& pl, const Work& w, hipStream_t) {
    ++g_launches;
    const size_t rows = pl.bf16_path ? (size_t)p.B * pl.splits * p.H : (size_t)p.B * p.H;
    memset(w.opart, 0, rows * 512 * act_bytes(pl));
    memset(w.lsepart, 0, rows * 4);
    return hipSuccess;
}

hipError_t launch_merge(const mla_decode_params_t&, const Plan&, const Work&, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_topk(int, int, int, const float*, long long, const int32_t*, int32_t*, long long, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_rope_apply(int, int, bool, bool, int, const void*, long long, long long, void*, long long,
                             long long, const int32_t*, const float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

}  // namespace mla
