// Device-side helpers shared by the Skiparse kernels: vector types, element
// conversion, and the 3D-RoPE cos/sin table that each workgroup builds in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skiparse_index.hpp"

namespace skiparse {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Element type tags (the public dtype codes).
struct BF16 {
    typedef uint16_t storage;
    static constexpr int kBytes = 2;
};
struct FP32 {
    typedef float storage;
    static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 (NaN stays NaN) through the hardware
// conversion instruction.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> one dword of two bf16 (low half = lo), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const f32x2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---------------------------------------------------------------------------
// 3D RoPE table
// ---------------------------------------------------------------------------
// Inverse frequencies 10000^(-2j/d_a) in fp64: inv[j] for the t axis (j < D/8, d_a = D/4),
// then inv[D/8 + j] for the h and w axes (j < 3D/16, d_a = 3D/8).  kRopeFreqs doubles.
template <int D>
struct RopeFreqs {
    static constexpr int kT = D / 8;
    static constexpr int kHW = 3 * D / 16;
    static constexpr int kCount = kT + kHW;
};

template <int D>
__device__ __forceinline__ void rope_inv_freqs(double* inv) {
    typedef RopeFreqs<D> F;
    for (int i = threadIdx.x; i < F::kCount; i += blockDim.x) {
        const bool t = i < F::kT;
        const int j = t ? i : i - F::kT;
        const double da = t ? (double)(D / 4) : (double)(3 * D / 8);
        inv[i] = pow(10000.0, -2.0 * (double)j / da);
    }
}

// (cos, sin) of pos * inv_freq: the angle is formed and reduced to [-pi, pi] in fp64 and
// evaluated with the fp32 sincos, within about one fp32 ulp of the fp64 values.
__device__ __forceinline__ float2 rope_cos_sin(int pos, double inv_freq) {
    const double theta = (double)pos * inv_freq;
    const double q = rint(theta * 0.15915494309189533577);     // 1 / (2 pi)
    const float r = (float)fma(-q, 6.2831853071795864769, theta);
    float sn, cs;
    sincosf(r, &sn, &cs);
    return make_float2(cs, sn);
}

// Layout (float2 = (cos, sin)):
//   [0, T*D/8)                      t axis: entry pos*(D/8) + j,    j < d_t/2 = D/8
//   [T*D/8, +H*3D/16)               h axis: entry pos*(3D/16) + j,  j < d_h/2 = 3D/16
//   [.., +W*3D/16)                  w axis: entry pos*(3D/16) + j,  j < d_w/2 = 3D/16
// Entry value: cos/sin of pos * 10000^(-2j/d_a) (rope_cos_sin).  `inv` is LDS scratch of
// RopeFreqs<D>::kCount doubles; the function ends with a workgroup barrier.
template <int D>
__device__ __forceinline__ void build_rope_table(float2* tab, int T, int H, int W, double* inv) {
    typedef RopeFreqs<D> F;
    rope_inv_freqs<D>(inv);
    __syncthreads();
    const int nt = T * F::kT, nh = H * F::kHW, nw = W * F::kHW;
    const int total = nt + nh + nw;
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        int pos, j;
        if (e < nt) {
            pos = e / F::kT; j = e - pos * F::kT;
        } else if (e < nt + nh) {
            const int r = e - nt; pos = r / F::kHW; j = F::kT + r - pos * F::kHW;
        } else {
            const int r = e - nt - nh; pos = r / F::kHW; j = F::kT + r - pos * F::kHW;
        }
        tab[e] = rope_cos_sin(pos, inv[j]);
    }
    __syncthreads();
}

// Offset of the table row of (axis, pos); entries j follow contiguously.
template <int D>
__device__ __forceinline__ int rope_row(int axis, int pos, int T, int H) {
    constexpr int kT = D / 8;
    constexpr int kHW = 3 * D / 16;
    if (axis == 0) return pos * kT;
    if (axis == 1) return T * kT + pos * kHW;
    return T * kT + H * kHW + pos * kHW;
}

// Rotate one rotate-half chunk pair in place: x1 (first half) and x2 (partner),
// CH elements each, using table entries row[j0 + e].
template <int CH>
__device__ __forceinline__ void rope_rotate(float (&x1)[CH], float (&x2)[CH], const float2* row) {
#pragma unroll
    for (int e = 0; e < CH; ++e) {
        const float2 cs = row[e];
        const float a = x1[e], b = x2[e];
        x1[e] = a * cs.x - b * cs.y;
        x2[e] = b * cs.x + a * cs.y;
    }
}

// Load CH consecutive elements of type E from global memory as floats.
template <typename E, int CH>
__device__ __forceinline__ void load_chunk_f32(const void* base, int64_t elem_off, float (&x)[CH]);

template <>
__device__ __forceinline__ void load_chunk_f32<BF16, 8>(const void* base, int64_t off, float (&x)[8]) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load_chunk_f32<BF16, 4>(const void* base, int64_t off, float (&x)[4]) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load_chunk_f32<FP32, 8>(const void* base, int64_t off, float (&x)[8]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
template <>
__device__ __forceinline__ void load_chunk_f32<FP32, 4>(const void* base, int64_t off, float (&x)[4]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i];
}

// Store CH floats as type E (bf16: round to nearest even).
template <typename E, int CH>
__device__ __forceinline__ void store_chunk_f32(void* base, int64_t elem_off, const float (&x)[CH]);

template <>
__device__ __forceinline__ void store_chunk_f32<BF16, 8>(void* base, int64_t off, const float (&x)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + off) = v;
}
template <>
__device__ __forceinline__ void store_chunk_f32<BF16, 4>(void* base, int64_t off, const float (&x)[4]) {
    u32x2 v;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + off) = v;
}
template <>
__device__ __forceinline__ void store_chunk_f32<FP32, 8>(void* base, int64_t off, const float (&x)[8]) {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off);
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = x[i]; b[i] = x[4 + i]; }
    p[0] = a;
    p[1] = b;
}
template <>
__device__ __forceinline__ void store_chunk_f32<FP32, 4>(void* base, int64_t off, const float (&x)[4]) {
    f32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = x[i];
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off) = a;
}

}  // namespace skiparse
