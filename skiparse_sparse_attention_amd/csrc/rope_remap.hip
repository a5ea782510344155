// Materialised Skiparse rearrange (with optional 3D RoPE) and its reverse.
//
// The Open-Sora Plan page ("Skiparse Attention", Single Skip / Group Skip
// implementations) applies add_rope to q and k, then rearranges q, k, v into
// (k*B, N/k, C) with the batch axis scope-major ('(k b)' / '(m b)'), and after
// attention applies reverse_sparse.  These kernels perform those data
// movements as standalone HBM-bound passes:
//
//   rope_remap_kernel: dst[(s*B + b)*L + p, head, :] = rope?(src[b, n(s,p), head, :])
//   reverse_kernel:    dst[b, n, head, :] = src[(s(n)*B + b)*L + p(n), head, :]
//
// Work decomposition: a flat grid-stride loop over (destination row, head,
// RoPE chunk pair) tasks.  Every task moves two head_dim/16-element chunks of
// one row (a chunk and its rotate-half partner), so a (row, head) record of
// head_dim elements is covered by 8 consecutive lanes and each wavefront reads
// and writes whole 256-byte head rows (bf16, head_dim 128).  Rows of one token
// are contiguous in both layouts, so source and destination accesses stay
// coalesced whatever the permutation.
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

template <int NB>
struct RawChunk;
template <>
struct RawChunk<8> { typedef u32x2 type; };
template <>
struct RawChunk<16> { typedef u32x4 type; };
template <>
struct RawChunk<32> { struct type { u32x4 a, b; }; };

template <int NB>
__device__ __forceinline__ void copy_raw(const void* src, void* dst, int64_t byte_off_src, int64_t byte_off_dst) {
    typedef typename RawChunk<NB>::type V;
    const V v = *reinterpret_cast<const V*>(reinterpret_cast<const char*>(src) + byte_off_src);
    *reinterpret_cast<V*>(reinterpret_cast<char*>(dst) + byte_off_dst) = v;
}

template <int D, typename E>
__global__ void __launch_bounds__(256) rope_remap_kernel(RemapParams a) {
    extern __shared__ float2 rope_tab[];
    constexpr int CH = D / 16;                    // elements per RoPE chunk
    constexpr int CB = CH * E::kBytes;            // bytes per RoPE chunk
    if (a.rope_mask) {
        build_rope_table<D>(rope_tab, a.T, a.H, a.W);
        __syncthreads();
    }
    const uint32_t tasks_per_row = (uint32_t)a.heads * 8u;
    const uint32_t total = (uint32_t)a.rows * tasks_per_row;
    const uint32_t HW = (uint32_t)a.H * (uint32_t)a.W;
    for (uint32_t g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
        const uint32_t row = g / tasks_per_row;        // destination row (s*B + b)*L + p
        const uint32_t task = g - row * tasks_per_row;
        const uint32_t head = task >> 3;
        const int cp = (int)(task & 7u);
        const uint32_t p = row % (uint32_t)a.L;
        const uint32_t sb = row / (uint32_t)a.L;
        const uint32_t s = sb / (uint32_t)a.B;
        const uint32_t b = sb - s * (uint32_t)a.B;
        const int64_t n = scope_token(p, s, a.k, a.mode);
        const int64_t src_elem = (((int64_t)b * a.N + n) * a.heads + head) * D;
        const int64_t dst_elem = ((int64_t)row * a.heads + head) * D;
        const RopePair rp = rope_pair(cp);
        const float2* trow = nullptr;
        if (a.rope_mask) {
            const uint32_t nn = (uint32_t)n;
            const uint32_t t = nn / HW;
            const uint32_t h = (nn / (uint32_t)a.W) % (uint32_t)a.H;
            const uint32_t w = nn % (uint32_t)a.W;
            const int pos = rp.axis == 0 ? (int)t : (rp.axis == 1 ? (int)h : (int)w);
            trow = rope_tab + rope_row<D>(rp.axis, pos, a.T, a.H) + rp.jchunk * CH;
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (i >= a.ntensors) break;
            const int64_t s1 = src_elem + rp.c1 * CH, s2 = src_elem + rp.c2 * CH;
            const int64_t d1 = dst_elem + rp.c1 * CH, d2 = dst_elem + rp.c2 * CH;
            if (a.rope_mask & (1 << i)) {
                float x1[CH], x2[CH];
                load_chunk_f32<E, CH>(a.src[i], s1, x1);
                load_chunk_f32<E, CH>(a.src[i], s2, x2);
                rope_rotate<CH>(x1, x2, trow);
                store_chunk_f32<E, CH>(a.dst[i], d1, x1);
                store_chunk_f32<E, CH>(a.dst[i], d2, x2);
            } else {
                copy_raw<CB>(a.src[i], a.dst[i], s1 * E::kBytes, d1 * E::kBytes);
                copy_raw<CB>(a.src[i], a.dst[i], s2 * E::kBytes, d2 * E::kBytes);
            }
        }
    }
}

// Reverse: one 16-byte piece per task; destination rows in original token order.
__global__ void __launch_bounds__(256) reverse_kernel(ReverseParams a) {
    const uint32_t pieces_per_row = a.row_bytes / 16u;
    const uint32_t total = (uint32_t)a.rows * pieces_per_row;
    for (uint32_t g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
        const uint32_t row = g / pieces_per_row;       // destination row b*N + n
        const uint32_t piece = g - row * pieces_per_row;
        const uint32_t b = row / (uint32_t)a.N;
        const uint32_t n = row - b * (uint32_t)a.N;
        int64_t s, p;
        token_scope(n, a.k, a.mode, &s, &p);
        const int64_t src_row = (s * a.B + b) * a.L + p;
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(a.src) + src_row * a.row_bytes + piece * 16u);
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.dst) + (int64_t)row * a.row_bytes + piece * 16u) = v;
    }
}

template <int D, typename E>
static hipError_t launch_remap_t(const RemapParams& a, hipStream_t stream, int grid) {
    const size_t lds = a.rope_mask ? (size_t)rope_table_pairs(a.T, a.H, a.W, D) * sizeof(float2) : 0;
    hipLaunchKernelGGL((rope_remap_kernel<D, E>), dim3(grid), dim3(256), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_rope_remap(const RemapParams& a, int head_dim, int dtype, hipStream_t stream, int grid) {
    if (head_dim == 128) {
        return dtype == 0 ? launch_remap_t<128, BF16>(a, stream, grid) : launch_remap_t<128, FP32>(a, stream, grid);
    }
    return dtype == 0 ? launch_remap_t<64, BF16>(a, stream, grid) : launch_remap_t<64, FP32>(a, stream, grid);
}

hipError_t launch_reverse(const ReverseParams& a, hipStream_t stream, int grid) {
    hipLaunchKernelGGL(reverse_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace skiparse
