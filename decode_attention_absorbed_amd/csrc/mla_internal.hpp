// Host-side plan and launch interface between the C API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {

// Launch plan of one decode call.
struct Plan {
    bool bf16_path;     // bf16 MFMA kernels (dtype_act bf16) or fp32 kernels
    int heads_per_wg;   // bf16 path: 32 * nhg heads per attention workgroup
    int nhg;            // bf16 path: 32-head groups per workgroup (1, 2 or 4)
    int hgroups;        // workgroups per (sequence, split) along heads
    int splits;         // split-KV partitions per sequence
    int tile_rows;      // rows gathered per attention iteration
};

// Carve-up of the caller's workspace.
struct Work {
    void* qt;           // Q~ [B][H][576] (bf16 or fp32)
    void* qlo;          // bf16 path: low bf16 parts of Q~'s rotary features [B][H][64]
    int32_t* list;      // compacted selection [B][K], ascending, 1-based (position + 1)
    int32_t* counts;    // selected rows per sequence [B]
    uint32_t* status;   // validation status word
    void* opart;        // split partials [H][B][S][512] (bf16; fp32 path: [B][H][512] fp32)
    float* lsepart;     // [H][B][S] log2-domain sum-exp of each partial (fp32 path: [B][H])
    size_t bytes;       // total bytes used
};

// Sets the calling thread's last error message; returns code.
int set_error(int code, const char* msg);

// Sizes of the workspace regions; returns the total (0 on overflow).
size_t workspace_layout(int B, int H, int K, bool bf16_path, int splits, void* base, Work* w);

hipError_t launch_rope_freqs(const mla_rope_cfg_t& cfg, float* table, hipStream_t s);
hipError_t launch_prep(const mla_decode_params_t& p, const Plan& plan, const Work& w, bool validate,
                       hipStream_t s);
hipError_t launch_attn(const mla_decode_params_t& p, const Plan& plan, const Work& w, hipStream_t s);
hipError_t launch_merge(const mla_decode_params_t& p, const Plan& plan, const Work& w, hipStream_t s);
hipError_t launch_topk(int B, int k, int max_len, const float* scores, long long score_stride,
                       const int32_t* cache_lens, int32_t* out, long long out_stride, hipStream_t s);
hipError_t launch_rope_apply(int N, int H, bool bf16_io, bool interleaved, int table_len,
                             const void* x, long long xs_n, long long xs_h,
                             void* y, long long ys_n, long long ys_h,
                             const int32_t* positions, const float* table, hipStream_t s);

}  // namespace mla
