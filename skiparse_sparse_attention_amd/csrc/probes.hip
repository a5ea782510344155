// Measurement aids, not part of the method: the two ceilings the attention and the memory
// passes are compared against, measured on the part itself rather than taken from its
// specification.
//
//   mfma_stream_kernel: bf16 32x32x16 matrix products and nothing else (no memory traffic in
//     the loop), four independent accumulator chains per wavefront so the matrix pipe never
//     waits on a result; 2*32*32*16 FLOP per product.
//   stream_copy_kernel: dst = src in 16-byte pieces, nontemporal loads and stores, a
//     grid-stride loop with four pieces per lane in flight -- the access pattern of the
//     RoPE / remap passes without their index and rotation arithmetic.
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void mfma_stream_kernel(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // small lane-dependent values: the products cannot be folded away, and stay finite
        a[e] = (__bf16)((float)((lane + e) & 7) * 0.125f);
        b[e] = (__bf16)((float)((lane * 3 + e) & 7) * 0.125f);
    }
    f32x16 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kProbeThreads) void stream_copy_kernel(const u32x4* src, u32x4* dst, int64_t pieces) {
    constexpr int kU = 4;
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    for (int64_t base = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; base < pieces; base += stride * kU) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t t = base + u * stride;
            v[u] = __builtin_nontemporal_load(src + (t < pieces ? t : pieces - 1));
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t t = base + u * stride;
            if (t < pieces) __builtin_nontemporal_store(v[u], dst + t);
        }
    }
}

}  // namespace

hipError_t launch_probe_mfma(int blocks, int iters, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_stream_kernel, dim3(blocks), dim3(kProbeThreads), 0, stream, iters, out);
    return hipGetLastError();
}

hipError_t launch_probe_stream(const void* src, void* dst, int64_t pieces, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), pieces);
    return hipGetLastError();
}

int probe_threads() { return kProbeThreads; }

}  // namespace skiparse
