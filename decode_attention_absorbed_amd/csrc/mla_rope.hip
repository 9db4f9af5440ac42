// Rotary embedding of 64-wide vectors at per-row positions, in either
// feature layout.  Source: page "Rotated query part", excerpt apply-rope:
// the features are taken as 32 complex pairs, each multiplied by
// (cos, sin)(t * theta'_i) from the rotation table; the attention path keeps
// the pairs interleaved ((2i, 2i+1)), the indexer keeps them split in two
// halves ((i, i+32): the vector is read as [2][32] and transposed, and the
// real parts come back first).
//
// Work unit: 8 pairs per thread, 4 threads per vector.  Interleaved: the
// thread owns 16 contiguous features; halves: 8 contiguous features in each
// half (16-byte accesses for bf16).  Each thread reads its features and
// their 8 (cos, sin) entries, then writes the same features, so y may alias x.  A position outside the
// table writes NaN to the whole vector.
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

struct RopeApplyArgs {
    long long NH;                  // vectors
    int H, interleaved, table_len;
    const void* x; long long xs_n, xs_h;
    void* y;       long long ys_n, ys_h;
    const int32_t* positions;
    const float* table;
};

// Eight consecutive elements as fp32 (16 or 32 bytes, aligned), and back.
template <typename T> __device__ __forceinline__ void ld8(const T* p, float (&v)[8]);
template <> __device__ __forceinline__ void ld8<bf16>(const bf16* p, float (&v)[8]) {
    const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
template <> __device__ __forceinline__ void ld8<float>(const float* p, float (&v)[8]) {
    const f32x4 x0 = *(const f32x4*)p, x1 = *(const f32x4*)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = x0[e]; v[4 + e] = x1[e]; }
}
template <typename T> __device__ __forceinline__ void st8(T* p, const float (&v)[8]);
template <> __device__ __forceinline__ void st8<bf16>(bf16* p, const float (&v)[8]) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f2bf(v[e]);
    *(bf16x8*)p = x;
}
template <> __device__ __forceinline__ void st8<float>(float* p, const float (&v)[8]) {
    f32x4 x0, x1;
#pragma unroll
    for (int e = 0; e < 4; ++e) { x0[e] = v[e]; x1[e] = v[4 + e]; }
    *(f32x4*)p = x0;
    *(f32x4*)(p + 4) = x1;
}

// Thread q (0..3) of a vector owns pairs 8q .. 8q+7.
template <typename T>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyArgs a) {
    const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long v = g >> 2;                  // vector
    if (v >= a.NH) return;
    const int q = (int)(g & 3);
    const long long n = v / a.H;
    const int h = (int)(v - n * a.H);
    const T* x = static_cast<const T*>(a.x) + n * a.xs_n + h * a.xs_h;
    T* y = static_cast<T*>(a.y) + n * a.ys_n + h * a.ys_h;
    const int t = a.positions[n];

    float re[8], im[8];                          // first and second members of the 8 pairs
    if (a.interleaved) {
        float lo[8], hi[8];
        ld8<T>(x + 16 * q, lo);
        ld8<T>(x + 16 * q + 8, hi);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            re[j] = lo[2 * j]; im[j] = lo[2 * j + 1];
            re[4 + j] = hi[2 * j]; im[4 + j] = hi[2 * j + 1];
        }
    } else {
        ld8<T>(x + 8 * q, re);
        ld8<T>(x + 32 + 8 * q, im);
    }
    float o_re[8], o_im[8];
    if (t >= 0 && t < a.table_len) {
        const f32x4* cs = reinterpret_cast<const f32x4*>(a.table + ((long long)t * 32 + 8 * q) * 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x4 c = cs[k];               // (cos, sin) of pairs 8q + 2k and 8q + 2k + 1
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = 2 * k + e;
                o_re[j] = re[j] * c[2 * e] - im[j] * c[2 * e + 1];
                o_im[j] = re[j] * c[2 * e + 1] + im[j] * c[2 * e];
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) o_re[j] = o_im[j] = __builtin_nanf("");
    }
    if (a.interleaved) {
        float lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo[2 * j] = o_re[j]; lo[2 * j + 1] = o_im[j];
            hi[2 * j] = o_re[4 + j]; hi[2 * j + 1] = o_im[4 + j];
        }
        st8<T>(y + 16 * q, lo);
        st8<T>(y + 16 * q + 8, hi);
    } else {
        st8<T>(y + 8 * q, o_re);
        st8<T>(y + 32 + 8 * q, o_im);
    }
}

hipError_t launch_rope_apply(int N, int H, bool bf16_io, bool interleaved, int table_len,
                             const void* x, long long xs_n, long long xs_h,
                             void* y, long long ys_n, long long ys_h,
                             const int32_t* positions, const float* table, hipStream_t s) {
    RopeApplyArgs a{(long long)N * H, H, interleaved ? 1 : 0, table_len, x, xs_n, xs_h, y, ys_n, ys_h,
                    positions, table};
    const long long threads = a.NH * 4;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (bf16_io) hipLaunchKernelGGL(rope_apply_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a);
    else         hipLaunchKernelGGL(rope_apply_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
