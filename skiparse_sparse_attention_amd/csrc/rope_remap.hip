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
// Work decomposition: one wavefront moves one whole token row (all heads) of a tensor at a
// time, in a grid-stride loop over destination rows (and tensors).  The row's scope, in-scope
// position, source token and grid position are wave-uniform scalar arithmetic done once per
// row; lanes then stream the row's bytes in 16-byte pieces.  A rotated tensor is processed
// as (head, RoPE chunk pair) tasks, one chunk and its rotate-half partner per task, so a
// lane holds both halves of every pair it rotates.  Token rows are contiguous in both
// layouts (heads*head_dim elements), so every access is part of a fully used 128-byte line.
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

// Copy `pieces` 16-byte pieces of one row with the 64 lanes of a wavefront, kU pieces per lane
// per round, all loads of a round issued before its stores.  Data is touched once, so loads
// and stores are nontemporal (streamed past the caches).
__device__ __forceinline__ void copy_row_pieces(const char* src, char* dst, int pieces, int lane) {
    constexpr int kU = 6;
    for (int t0 = 0; t0 < pieces; t0 += 64 * kU) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + min(t0 + 64 * u + lane, pieces - 1) * 16));
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = t0 + 64 * u + lane;
            if (t < pieces) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + t * 16));
        }
    }
}

// One destination row of one bf16 tensor at head_dim 128, where a RoPE chunk is exactly one
// 16-byte piece.  Lane l moves piece t (head t / 16, chunk c = t % 16), so each load and store
// of a wavefront covers four whole head rows; the loads of a round are all issued before its
// stores.  The rotate-half partner chunk of c lies 2 (t axis) or 3 (h, w axes) chunks away in
// the same head row, i.e. in a lane of the same group of 16; its bytes are fetched with a
// cross-lane permute.  A first-half chunk computes x c - y s and its partner y c + x s, from
// the same (cos, sin) entries.
__device__ __forceinline__ void rope_row_bf16_d128(const char* src, char* dst, int pieces, int lane,
                                                   const float2* tab, int T, int H, const int (&pos)[3]) {
    constexpr int D = 128, CH = 8;
    constexpr int kU = 6;
    const int c = lane & 15;
    // chunk -> partner offset, role, axis, frequency block (the pairs of rope_pair, by chunk)
    const int axis = c < 4 ? 0 : (c < 10 ? 1 : 2);
    const int first = axis == 0 ? (c < 2) : (axis == 1 ? (c < 7) : (c < 13));
    const int delta = axis == 0 ? 2 : 3;
    const int partner = lane + (first ? delta : -delta);
    const int jchunk = axis == 0 ? (c & 1) : (axis == 1 ? (c - 4) % 3 : (c - 10) % 3);
    const float2* trow = tab + rope_row<D>(axis, pos[axis], T, H) + jchunk * CH;
    const float sgn = first ? -1.f : 1.f;
    for (int t0 = 0; t0 < pieces; t0 += 64 * kU) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + min(t0 + 64 * u + lane, pieces - 1) * 16));
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            u32x4 w, o;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner * 4, (int)v[u][q]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 cs0 = trow[2 * q], cs1 = trow[2 * q + 1];
                const float x0 = __uint_as_float(v[u][q] << 16), x1 = __uint_as_float(v[u][q] & 0xffff0000u);
                const float y0 = __uint_as_float(w[q] << 16), y1 = __uint_as_float(w[q] & 0xffff0000u);
                o[q] = pack_bf16x2(x0 * cs0.x + sgn * (y0 * cs0.y), x1 * cs1.x + sgn * (y1 * cs1.y));
            }
            const int t = t0 + 64 * u + lane;
            if (t < pieces) __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + t * 16));
        }
    }
}

template <int D, typename E>
__global__ void __launch_bounds__(256) rope_remap_kernel(RemapParams a) {
    extern __shared__ float2 rope_tab[];
    constexpr int CH = D / 16;                    // elements per RoPE chunk
    if (a.rope_mask)
        build_rope_table<D>(rope_tab, a.T, a.H, a.W,
                            reinterpret_cast<double*>(rope_tab + rope_table_pairs(a.T, a.H, a.W, D)));
    const int lane = threadIdx.x & 63;
    const int nwaves = gridDim.x * (blockDim.x >> 6);
    const int wave0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
    const int row_elems = a.heads * D;
    const int64_t row_bytes = (int64_t)row_elems * E::kBytes;
    const int pairs = a.heads * 8;                // (head, chunk pair) tasks per row
    const int pieces = (int)(row_bytes / 16);     // 16-byte pieces per row
    if constexpr (D == 128 && E::kBytes == 2) {
        // units of work: (destination row, tensor), so the grid stays balanced to within one
        // row of one tensor
        const int units = a.rows * a.ntensors;
        for (int u = wave0; u < units; u += nwaves) {
            const int row = u / a.ntensors;
            const int i = u - row * a.ntensors;
            const int p = row % a.L;
            const int sb = row / a.L;
            const int s = sb / a.B;
            const int b = sb - s * a.B;
            const int n = (int)scope_token(p, s, a.k, a.mode);
            const char* src = reinterpret_cast<const char*>(a.src[i]) + ((int64_t)b * a.N + n) * row_bytes;
            char* dst = reinterpret_cast<char*>(a.dst[i]) + (int64_t)row * row_bytes;
            if ((a.rope_mask >> i) & 1) {
                const int pos[3] = {n / (a.H * a.W), (n / a.W) % a.H, n % a.W};
                rope_row_bf16_d128(src, dst, pieces, lane, rope_tab, a.T, a.H, pos);
            } else {
                copy_row_pieces(src, dst, pieces, lane);
            }
        }
        return;
    }
    for (int row = wave0; row < a.rows; row += nwaves) {   // destination row (s*B + b)*L + p
        const int p = row % a.L;
        const int sb = row / a.L;
        const int s = sb / a.B;
        const int b = sb - s * a.B;
        const int n = (int)scope_token(p, s, a.k, a.mode);
        const int64_t src_row = ((int64_t)b * a.N + n) * row_bytes;
        const int64_t dst_row = (int64_t)row * row_bytes;
        // grid position of the source token (for the RoPE table rows)
        const int pos_t = n / (a.H * a.W), pos_h = (n / a.W) % a.H, pos_w = n % a.W;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (i >= a.ntensors) break;
            const char* src = reinterpret_cast<const char*>(a.src[i]) + src_row;
            char* dst = reinterpret_cast<char*>(a.dst[i]) + dst_row;
            if (a.rope_mask & (1 << i)) {
                // kU tasks per lane per round; the loads of a round are all issued before
                // its first store (indices past the row end are clamped for the loads and
                // their stores skipped)
                constexpr int kU = 4;
                for (int t0 = 0; t0 < pairs; t0 += 64 * kU) {
                    float x1[kU][CH], x2[kU][CH];
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int t = min(t0 + 64 * u + lane, pairs - 1);
                        const RopePair rp = rope_pair(t & 7);
                        const int64_t e = (int64_t)(t >> 3) * D;
                        load_chunk_f32<E, CH>(src, e + rp.c1 * CH, x1[u]);
                        load_chunk_f32<E, CH>(src, e + rp.c2 * CH, x2[u]);
                    }
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int t = t0 + 64 * u + lane;
                        if (t < pairs) {
                            const RopePair rp = rope_pair(t & 7);
                            const int pos = rp.axis == 0 ? pos_t : (rp.axis == 1 ? pos_h : pos_w);
                            rope_rotate<CH>(x1[u], x2[u], rope_tab + rope_row<D>(rp.axis, pos, a.T, a.H) + rp.jchunk * CH);
                            const int64_t e = (int64_t)(t >> 3) * D;
                            store_chunk_f32<E, CH>(dst, e + rp.c1 * CH, x1[u]);
                            store_chunk_f32<E, CH>(dst, e + rp.c2 * CH, x2[u]);
                        }
                    }
                }
            } else {
                copy_row_pieces(src, dst, pieces, lane);
            }
        }
    }
}

// Reverse: one wavefront per destination row (original token order), 16-byte pieces.
__global__ void __launch_bounds__(256) reverse_kernel(ReverseParams a) {
    const int lane = threadIdx.x & 63;
    const int nwaves = gridDim.x * (blockDim.x >> 6);
    const int wave0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)));
    const int pieces = (int)(a.row_bytes / 16u);
    for (int row = wave0; row < a.rows; row += nwaves) {   // destination row b*N + n
        const int b = row / a.N;
        const int n = row - b * a.N;
        int64_t s, p;
        token_scope(n, a.k, a.mode, &s, &p);
        const char* src = reinterpret_cast<const char*>(a.src) + ((s * a.B + b) * a.L + p) * (int64_t)a.row_bytes;
        char* dst = reinterpret_cast<char*>(a.dst) + (int64_t)row * a.row_bytes;
        copy_row_pieces(src, dst, pieces, lane);
    }
}

template <int D, typename E>
static hipError_t launch_remap_t(const RemapParams& a, hipStream_t stream, int grid) {
    const size_t lds =
        a.rope_mask ? (size_t)rope_table_pairs(a.T, a.H, a.W, D) * sizeof(float2) + RopeFreqs<D>::kCount * sizeof(double) : 0;
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
