// Rotary embedding of 64-wide vectors at per-row positions, in either
// feature layout.  Source: page "Rotated query part", excerpt apply-rope:
// the features are taken as 32 complex pairs, each multiplied by
// (cos, sin)(t * theta'_i) from the rotation table; the attention path keeps
// the pairs interleaved ((2i, 2i+1)), the indexer keeps them split in two
// halves ((i, i+32): the vector is read as [2][32] and transposed, and the
// real parts come back first).
//
// Work unit: 4 pairs per thread, 8 threads per vector.  Interleaved: the
// thread owns 8 contiguous features; halves: 4 contiguous features in each
// half.  Each thread reads its features and the 4 (cos, sin) entries, then
// writes the same features, so y may alias x.  A position outside the
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

template <typename T> struct Vec4;
template <> struct Vec4<bf16>  { using type = bf16x4; };
template <> struct Vec4<float> { using type = float4; };

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
    const auto r = *reinterpret_cast<const typename Vec4<T>::type*>(p);
    v[0] = to_f32<T>(r[0]); v[1] = to_f32<T>(r[1]); v[2] = to_f32<T>(r[2]); v[3] = to_f32<T>(r[3]);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float (&v)[4]) {
    const float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]) {
    typename Vec4<T>::type r;
    r[0] = from_f32<T>(v[0]); r[1] = from_f32<T>(v[1]); r[2] = from_f32<T>(v[2]); r[3] = from_f32<T>(v[3]);
    *reinterpret_cast<typename Vec4<T>::type*>(p) = r;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void rope_apply_kernel(RopeApplyArgs a) {
    const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long v = g >> 3;                  // vector
    if (v >= a.NH) return;
    const int part = (int)(g & 7);               // pairs 4 part .. 4 part + 3
    const long long n = v / a.H;
    const int h = (int)(v - n * a.H);
    const T* x = static_cast<const T*>(a.x) + n * a.xs_n + h * a.xs_h;
    T* y = static_cast<T*>(a.y) + n * a.ys_n + h * a.ys_h;
    const int t = a.positions[n];

    // first and second members of the 4 pairs
    float re[4], im[4];
    if (a.interleaved) {
        float lo[4], hi[4];
        load4<T>(x + 8 * part, lo);
        load4<T>(x + 8 * part + 4, hi);
        re[0] = lo[0]; im[0] = lo[1]; re[1] = lo[2]; im[1] = lo[3];
        re[2] = hi[0]; im[2] = hi[1]; re[3] = hi[2]; im[3] = hi[3];
    } else {
        load4<T>(x + 4 * part, re);
        load4<T>(x + 32 + 4 * part, im);
    }
    float o_re[4], o_im[4];
    if (t >= 0 && t < a.table_len) {
        const float4* cs = reinterpret_cast<const float4*>(a.table + ((long long)t * 32 + 4 * part) * 2);
        const float4 c01 = cs[0], c23 = cs[1];   // (cos, sin) of pairs 4 part + {0, 1}, then {2, 3}
        const float c[4] = {c01.x, c01.z, c23.x, c23.z};
        const float s[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o_re[j] = re[j] * c[j] - im[j] * s[j];
            o_im[j] = re[j] * s[j] + im[j] * c[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) o_re[j] = o_im[j] = __builtin_nanf("");
    }
    if (a.interleaved) {
        const float lo[4] = {o_re[0], o_im[0], o_re[1], o_im[1]};
        const float hi[4] = {o_re[2], o_im[2], o_re[3], o_im[3]};
        store4<T>(y + 8 * part, lo);
        store4<T>(y + 8 * part + 4, hi);
    } else {
        store4<T>(y + 4 * part, o_re);
        store4<T>(y + 32 + 4 * part, o_im);
    }
}

hipError_t launch_rope_apply(int N, int H, bool bf16_io, bool interleaved, int table_len,
                             const void* x, long long xs_n, long long xs_h,
                             void* y, long long ys_n, long long ys_h,
                             const int32_t* positions, const float* table, hipStream_t s) {
    RopeApplyArgs a{(long long)N * H, H, interleaved ? 1 : 0, table_len, x, xs_n, xs_h, y, ys_n, ys_h,
                    positions, table};
    const long long threads = a.NH * 8;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (bf16_io) hipLaunchKernelGGL(rope_apply_kernel<bf16>, dim3(blocks), dim3(256), 0, s, a);
    else         hipLaunchKernelGGL(rope_apply_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mla
