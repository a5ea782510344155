// Materialised Skiparse rearrange (with optional 3D RoPE) and its reverse.
//
// The Open-Sora Plan page ("Skiparse Attention", Single Skip and Group Skip code) rotates q
// and k, regroups q, k, v into k scopes -- a (k*B, N/k, C) tensor whose row s*B + b holds
// scope s of batch b -- and after attention moves every row back to its token.  These
// kernels perform those data movements as standalone HBM-bound passes:
//
//   rope_remap_*:   dst[(s*B + b)*L + p, head, :] = rope?(src[b, n(s,p), head, :])
//   reverse_kernel: dst[b, n, head, :] = src[(s(n)*B + b)*L + p(n), head, :]
//
// Work decomposition: one wavefront moves one whole token row (all heads) at a time; the
// row's scope, in-scope position, source token and grid position are wave-uniform scalar
// arithmetic done once per row, and lanes stream the row's bytes in 16-byte pieces.  At
// bf16 / head_dim 128 (the measured path) a wavefront moves one destination row of every
// tensor in a one-shot grid, evaluating the source token's RoPE pairs itself; other
// combinations loop over rows with the whole table in LDS and rotate (head, chunk pair)
// tasks.  Token rows are contiguous in both layouts (heads*head_dim elements), so every
// access is part of a fully used 128-byte line.
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

// The token's 64 (cos, sin) pairs at head_dim 128, one per lane (t axis pairs 0-15 with
// d_t = 32, h axis 16-39 and w axis 40-63 with d = 48): float64 angle and sincos, rounded to
// float32 -- the values of the attention kernels' tables.
__device__ __forceinline__ float2 token_pair_d128(int lane, int n, int H, int W) {
    const int axis = lane < 16 ? 0 : (lane < 40 ? 1 : 2);
    const int j = lane - (axis == 0 ? 0 : (axis == 1 ? 16 : 40));
    const int pos = axis == 0 ? n / (H * W) : (axis == 1 ? (n / W) % H : n % W);
    const double da = axis == 0 ? 32.0 : 48.0;
    const double theta = (double)pos * pow(10000.0, -2.0 * (double)j / da);
    double sn, cs;
    sincos(theta, &sn, &cs);
    return make_float2((float)cs, (float)sn);
}

// bf16, head_dim 128 (the measured path): one wavefront per destination row, moving that row
// of every tensor; a one-shot grid (no loop over rows).  Lane l moves the 16-byte pieces
// l, l + 64, ... of each row, all of RoPE chunk c = l % 16, so its eight (cos, sin) pairs are
// fixed.  The first round's loads of every tensor are issued before the source token's pairs
// are evaluated (one per lane); the rotate-half partner chunk (2 or 3 chunks away in the same
// head row, a lane of the same group of 16) comes through a cross-lane permute, and a first-half
// chunk computes x c - y s, its partner y c + x s.  Loads and stores are nontemporal (data is
// touched once).
constexpr int kRemapWaves = 4;

__global__ void __launch_bounds__(64 * kRemapWaves) rope_remap_row_kernel(RemapParams a) {
    constexpr int CH = 8, kU = 6;
    __shared__ __attribute__((aligned(16))) float2 pairs[kRemapWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kRemapWaves + wave));
    if (row >= a.rows) return;
    const int64_t row_bytes = (int64_t)a.heads * 128 * 2;
    const int pieces = a.heads * 16;
    const int p = row % a.L;
    const int sb = row / a.L;
    const int s = sb / a.B;
    const int b = sb - s * a.B;
    const int n = (int)scope_token(p, s, a.k, a.mode);
    const char* src[3];
    char* dst[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        src[i] = reinterpret_cast<const char*>(a.src[i]) + ((int64_t)b * a.N + n) * row_bytes;
        dst[i] = reinterpret_cast<char*>(a.dst[i]) + (int64_t)row * row_bytes;
    }
    // chunk -> partner offset, role, axis, frequency block (the pairs of rope_pair, by chunk)
    const int c = lane & 15;
    const int axis = c < 4 ? 0 : (c < 10 ? 1 : 2);
    const bool first = axis == 0 ? (c < 2) : (axis == 1 ? (c < 7) : (c < 13));
    const int delta = axis == 0 ? 2 : 3;
    const int partner = lane + (first ? delta : -delta);
    const int jchunk = axis == 0 ? (c & 1) : (axis == 1 ? (c - 4) % 3 : (c - 10) % 3);
    const float sgn = first ? -1.f : 1.f;
    u32x4 v[3][kU];
    auto load_round = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (i >= a.ntensors) break;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                v[i][u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(src[i] + min(t0 + 64 * u + lane, pieces - 1) * 16));
        }
    };
    load_round(0);
    float2 cs[CH];
    if (a.rope_mask) {
        pairs[wave][lane] = token_pair_d128(lane, n, a.H, a.W);
        __builtin_amdgcn_wave_barrier();
        const float2* trow = pairs[wave] + (axis == 0 ? 0 : (axis == 1 ? 16 : 40)) + jchunk * CH;
#pragma unroll
        for (int e = 0; e < CH; ++e) cs[e] = trow[e];
    }
    for (int t0 = 0; t0 < pieces; t0 += 64 * kU) {
        if (t0 > 0) load_round(t0);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (i >= a.ntensors) break;
            const bool rot = (a.rope_mask >> i) & 1;
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                u32x4 o = v[i][u];
                if (rot) {
                    u32x4 w;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner * 4, (int)v[i][u][q]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float2 cs0 = cs[2 * q], cs1 = cs[2 * q + 1];
                        const float x0 = __uint_as_float(v[i][u][q] << 16), x1 = __uint_as_float(v[i][u][q] & 0xffff0000u);
                        const float y0 = __uint_as_float(w[q] << 16), y1 = __uint_as_float(w[q] & 0xffff0000u);
                        o[q] = pack_bf16x2(x0 * cs0.x + sgn * (y0 * cs0.y), x1 * cs1.x + sgn * (y1 * cs1.y));
                    }
                }
                const int t = t0 + 64 * u + lane;
                if (t < pieces) __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst[i] + t * 16));
            }
        }
    }
}

// Other head_dim / dtype combinations: (head, chunk pair) tasks, a grid-stride loop over
// destination rows, and the whole table built in LDS by every workgroup.
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
    if constexpr (D == 128 && E::kBytes == 2) {
        const int64_t blocks = ((int64_t)a.rows + kRemapWaves - 1) / kRemapWaves;
        hipLaunchKernelGGL(rope_remap_row_kernel, dim3((unsigned)blocks), dim3(64 * kRemapWaves), 0, stream, a);
        return hipGetLastError();
    }
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
