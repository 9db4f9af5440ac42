// Device-side helpers shared by the MLA decode kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define MLA_LDS __attribute__((address_space(3)))

constexpr int D_NOPE = 128;
constexpr int D_ROPE = 64;
constexpr int D_V = 128;
constexpr int RANK = 512;
constexpr int ROW = RANK + D_ROPE;       // 576 features per cached position
constexpr int ROW_CHUNKS = ROW / 8;      // 72 chunks of 16 bytes (8 bf16)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Validation status bits (mirror MLA_BAD_* in the public header).
constexpr uint32_t BAD_INDEX_RANGE = 1u, BAD_DUPLICATE = 2u, BAD_EMPTY = 4u, BAD_CACHE_LEN = 8u;

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }   // round to nearest even

// v_mfma_f32_32x32x16_bf16.  Lane l holds A[m = l%32][k = 8*(l/32) + j] and
// B[k = 8*(l/32) + j][n = l%32] (j < 8); the result lane l holds
// D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32] for i < 16.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane block, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const MLA_LDS void* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Copy 16 bytes per lane from global memory straight into LDS: lane l's
// bytes land at lds_base + 16*l (lds_base must be wave-uniform).
__device__ __forceinline__ void global_to_lds16(const void* src, MLA_LDS void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer -> LDS copy (buffer_load ... lds): lane l writes its `size` bytes at
// lds_base + size * l.  lds_base must be wave-uniform.  Unlike the global
// form, the compiler does not treat the buffer form as a possible LDS access
// through FLAT, so LDS reads issued while such copies are in flight keep
// exact lgkmcnt waits.
__device__ __forceinline__ void buffer_to_lds16(rsrc_t r, uint32_t voff, MLA_LDS void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds4(rsrc_t r, uint32_t voff, MLA_LDS void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N): wait until at most N vector memory loads of this wave
// (global->LDS copies included) are outstanding.  gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | 0x0F70);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Load 8 consecutive weights/activations as bf16 (converting from fp32 when
// the source is fp32).
template <typename T> __device__ __forceinline__ bf16x8 load8_bf16(const T* p);
template <> __device__ __forceinline__ bf16x8 load8_bf16<bf16>(const bf16* p) {
    return *(const bf16x8*)p;
}
template <> __device__ __forceinline__ bf16x8 load8_bf16<float>(const float* p) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    return bf16x8{f2bf(a[0]), f2bf(a[1]), f2bf(a[2]), f2bf(a[3]),
                  f2bf(b[0]), f2bf(b[1]), f2bf(b[2]), f2bf(b[3])};
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return f2bf(x); }

}  // namespace mla
