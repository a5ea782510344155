// 8-bit operands of Skiparse attention for gfx950 (CDNA4).
//
// Wan 2.1 report, section 4.4.3 "Quantization" (paragraph "8-Bit FlashAttention"): the scores
// S = Q K^T are formed from Int8 operands and O = P V from FP8 (E4M3) operands.  This pass
// prepares Q, K and V for the 8-bit attention kernel (attn8_fwd.hip); the P operand is
// quantised inside that kernel.
//
//   q' = RoPE(q), k' = RoPE(k): float32 from a float32 cos/sin table (angles and their
//        cosines evaluated in float64, then rounded), one rounding per product and per
//        sum (no fused multiply-add), the same 3D RoPE as the bf16 path;
//   q8 = round_half_even(q' * (127 / q_amax)), q_amax = max |q'| over the head row
//        (one scale per batch, token and head);
//   k8 = round_half_even(k' * (127 / k_amax)), k_amax = max |k'| over every token and
//        channel of a (batch, head);
//   vt8 = E4M3(v * (448 / v_amax)), v_amax = max |v| over the tokens of a (batch, head,
//        channel), stored transposed per scope: vt8[b][head][s][c][p] for scope position p
//        (rows padded with zero codes to Lp = L rounded up to 64 keys).
// The reciprocals and products are float32 operations with one rounding each, so the integer
// codes are a function of the inputs alone.  A zero amax gives zero codes.
//
// Three launches: a fill of the amax outputs with zeros, a statistics pass that folds
// per-workgroup maxima of |k'| and |v| into k_amax and v_amax with atomic maxima (the bit
// patterns of non-negative floats order like unsigned integers), and the quantisation pass,
// one workgroup task per (batch, head, scope, 64 scope positions), which also transposes V
// through LDS.  Both passes issue a lane's loads for several rows (the quantisation pass: all
// of a task's q, k and v pieces) before using any of them: one row at a time left them
// latency-bound at about half the HBM rate.
#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

using namespace attn;

namespace {

constexpr int kD = 128;                // head_dim of the 8-bit path
constexpr int kCH = kD / 16;           // elements per RoPE chunk (rope_pair's chunk layout)
constexpr int kQ8Threads = 256;        // 4 wavefronts
constexpr int kQ8Tile = 64;            // scope positions per quantisation task
constexpr int kStatTokens = 512;       // tokens per statistics workgroup
constexpr int kQ8MaxGrid = 1024;       // quantisation workgroups (each builds the table once)
constexpr int kVtQuad = 128 * 4 + 16;  // bytes per row quad of the V codes in LDS: a dword
                                       // (4 rows) per channel, then a pad granule

typedef float f32x8 __attribute__((ext_vector_type(8)));

// x1' = x1 c - x2 s, x2' = x2 c + x1 s with every product and sum rounded to float32
__device__ __forceinline__ void rotate_rn(float x1, float x2, float c, float s, float& y1, float& y2) {
#pragma clang fp contract(off)
    y1 = x1 * c - x2 * s;
    y2 = x2 * c + x1 * s;
}

// int8 code of x * r (r = 127 / amax), the product rounded to float32, then to nearest even
__device__ __forceinline__ uint32_t int8_code(float x, float r) {
#pragma clang fp contract(off)
    const float y = __builtin_rintf(x * r);
    return (uint32_t)(int)fminf(fmaxf(y, -127.f), 127.f) & 0xffu;
}

// The raw chunk pair cp of the head row at `off`: chunk rp.c1 and its rotate-half partner
// rp.c2 (the loads only, so that a lane can have several rows' loads in flight).
template <typename E>
__device__ __forceinline__ void load_pair(__amdgpu_buffer_rsrc_t r, int off, const RopePair& rp,
                                          ChunkRaw<E, kCH>& w1, ChunkRaw<E, kCH>& w2) {
    buffer_load_dwords(r, off + rp.c1 * kCH * E::kBytes, w1.w);
    buffer_load_dwords(r, off + rp.c2 * kCH * E::kBytes, w2.w);
}

// A loaded chunk pair turned by RoPE at grid position q: x1 gets chunk rp.c1, x2 its partner.
template <typename E>
__device__ __forceinline__ void rotate_pair(const ChunkRaw<E, kCH>& w1, const ChunkRaw<E, kCH>& w2, const RopePair& rp,
                                            const char* tab, int T, int H, const Pos& q, float (&x1)[kCH],
                                            float (&x2)[kCH]) {
    raw_to_f32(w1, x1);
    raw_to_f32(w2, x2);
    const int pos = rp.axis == 0 ? q.t : (rp.axis == 1 ? q.h : q.w);
    const float* cs = reinterpret_cast<const float*>(tab + rope_tab_offset<kD>(T, H, rp.axis, pos, rp.jchunk * kCH, 0));
    float c[2 * kCH];
#pragma unroll
    for (int i = 0; i < kCH / 2; ++i) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(cs + 4 * i);
        c[4 * i] = v[0]; c[4 * i + 1] = v[1]; c[4 * i + 2] = v[2]; c[4 * i + 3] = v[3];
    }
#pragma unroll
    for (int e = 0; e < kCH; ++e) rotate_rn(x1[e], x2[e], c[2 * e], c[2 * e + 1], x1[e], x2[e]);
}

__device__ __forceinline__ Pos grid_pos(int n, int H, int W) {
    Pos q;
    q.t = n / (H * W); q.h = (n / W) % H; q.w = n % W;
    return q;
}

// kCH int8 codes packed little-endian into two dwords
__device__ __forceinline__ u32x2 pack_codes(const float (&x)[kCH], float r) {
    u32x2 w = {0u, 0u};
#pragma unroll
    for (int e = 0; e < kCH; ++e) w[e / 4] |= int8_code(x[e], r) << (8 * (e % 4));
    return w;
}

__global__ void __launch_bounds__(kQ8Threads) q8_fill_kernel(float* k_amax, float* v_amax, int nk, int nv) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nk + nv; i += gridDim.x * blockDim.x) {
        if (i < nk) k_amax[i] = 0.f;
        else v_amax[i - nk] = 0.f;
    }
}

// Statistics: workgroup (token chunk, batch * heads + head).  k: 8 lanes per token row, one
// RoPE chunk pair each; v: 16 lanes per token row, one 8-channel chunk each.  Partial maxima
// meet in LDS, then one atomic maximum per channel (and one for k) per workgroup.
template <typename E>
__global__ void __launch_bounds__(kQ8Threads) q8_stats_kernel(Q8Params a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int ES = E::kBytes;
    char* tab = lds;
    float* red = reinterpret_cast<float*>(lds + (a.T + a.H + a.W) * 256);   // [kQ8Threads / 16][kD], then k
    const int bh = blockIdx.y, b = bh / a.heads, head = bh % a.heads;
    const int tid = threadIdx.x;
    const int row_bytes = a.heads * kD * ES;
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * kD * ES;
    const int slice_bytes = a.N * row_bytes - head * kD * ES;
    const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
    build_banked_rope_table<kD>(tab, a.T, a.H, a.W, 0);
    __syncthreads();
    const int n0 = blockIdx.x * kStatTokens;
    const int n1 = min(n0 + kStatTokens, a.N);
    // k: row tid / 8 of each 32-row step, chunk pair tid % 8; kStatK steps' loads are issued
    // before any of them is used (rows past n1 read as zeros through the buffer range, and
    // zeros leave the maxima unchanged)
    constexpr int kStatK = 4, kStatV = 8;
    const RopePair rp = rope_pair(tid & 7);
    float km = 0.f;
    for (int n = n0 + (tid >> 3); n < n1; n += kStatK * (kQ8Threads / 8)) {
        ChunkRaw<E, kCH> w1[kStatK], w2[kStatK];
#pragma unroll
        for (int i = 0; i < kStatK; ++i) {
            const int ni = n + i * (kQ8Threads / 8);
            load_pair<E>(kbuf, (ni < n1 ? ni : a.N) * row_bytes, rp, w1[i], w2[i]);
        }
#pragma unroll
        for (int i = 0; i < kStatK; ++i) {
            const int ni = n + i * (kQ8Threads / 8);
            float x1[kCH], x2[kCH];
            rotate_pair<E>(w1[i], w2[i], rp, tab, a.T, a.H, grid_pos(min(ni, a.N - 1), a.H, a.W), x1, x2);
#pragma unroll
            for (int e = 0; e < kCH; ++e) km = fmaxf(km, fmaxf(fabsf(x1[e]), fabsf(x2[e])));
        }
    }
    // v: row tid / 16 of each 16-row step, channels 8 (tid % 16) + [0, 8), kStatV steps' loads
    // in flight at a time
    const int vc = tid & 15;
    float vm[kCH];
#pragma unroll
    for (int e = 0; e < kCH; ++e) vm[e] = 0.f;
    for (int n = n0 + (tid >> 4); n < n1; n += kStatV * (kQ8Threads / 16)) {
        ChunkRaw<E, kCH> w[kStatV];
#pragma unroll
        for (int i = 0; i < kStatV; ++i) {
            const int ni = n + i * (kQ8Threads / 16);
            buffer_load_dwords(vbuf, (ni < n1 ? ni : a.N) * row_bytes + vc * kCH * ES, w[i].w);
        }
#pragma unroll
        for (int i = 0; i < kStatV; ++i) {
            float x[kCH];
            raw_to_f32(w[i], x);
#pragma unroll
            for (int e = 0; e < kCH; ++e) vm[e] = fmaxf(vm[e], fabsf(x[e]));
        }
    }
    float* wr = red + (tid >> 4) * kD + vc * kCH;
#pragma unroll
    for (int e = 0; e < kCH; ++e) wr[e] = vm[e];
    float* kred = red + (kQ8Threads / 16) * kD;
    {
        float m = km;
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
        if ((tid & 63) == 0) kred[tid >> 6] = m;
    }
    __syncthreads();
    if (tid < kD) {
        float m = 0.f;
        for (int r = 0; r < kQ8Threads / 16; ++r) m = fmaxf(m, red[r * kD + tid]);
        atomicMax(reinterpret_cast<unsigned*>(a.v_amax) + (int64_t)bh * kD + tid, __float_as_uint(m));
    } else if (tid == kD) {
        float m = 0.f;
        for (int r = 0; r < kQ8Threads / 64; ++r) m = fmaxf(m, kred[r]);
        atomicMax(reinterpret_cast<unsigned*>(a.k_amax) + bh, __float_as_uint(m));
    }
}

// Quantisation: task (batch, head, scope, tile of 64 scope positions).  q and k: 8 lanes per
// row, one RoPE chunk pair each (the q row's amax across the 8 lanes), codes stored as two
// 8-byte pieces straight to the token's row; v: lane l of a wave holds channels 2 l, 2 l + 1
// of four consecutive rows (so each load instruction of a wave reads one whole V head row),
// packs the codes of the four rows of each channel into one dword and writes both dwords
// into LDS, laid out row quad by row quad ([quad][channel] dwords, the quads 528 bytes
// apart); the vt8 rows are then gathered from there, four dwords per 16-byte piece.  Both LDS
// passes touch 64 distinct banks per instruction (the byte-wise transpose this replaced spent
// most of its LDS cycles in bank conflicts).
template <typename E>
__global__ void __launch_bounds__(kQ8Threads) q8_quant_kernel(Q8Params a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int ES = E::kBytes;
    char* tab = lds;
    char* vt = lds + (a.T + a.H + a.W) * 256;
    const int tid = threadIdx.x;
    const int row_bytes = a.heads * kD * ES;
    const int row8 = a.heads * kD;                              // bytes per token of q8 / k8
    const int L = a.N / a.sparse_k;
    const int tiles = a.Lp / kQ8Tile;
    const int tasks = a.B * a.heads * a.sparse_k * tiles;
    build_banked_rope_table<kD>(tab, a.T, a.H, a.W, 0);
    __syncthreads();
    const int cp = tid & 7;
    const RopePair rp = rope_pair(cp);
    const int vch = 2 * (tid & 63);          // this lane's V channel pair
    for (int task = blockIdx.x; task < tasks; task += gridDim.x) {
        const int pt = task % tiles;
        const int s = (task / tiles) % a.sparse_k;
        const int bh = task / (tiles * a.sparse_k);
        const int b = bh / a.heads, head = bh % a.heads;
        const int64_t slice = ((int64_t)b * a.N * a.heads + head) * kD * ES;
        const int slice_bytes = a.N * row_bytes - head * kD * ES;
        const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.q) + slice), (short)0, slice_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
        const int64_t slice8 = ((int64_t)b * a.N * a.heads + head) * kD;
        const int slice8_bytes = a.N * row8 - head * kD;
        const __amdgpu_buffer_rsrc_t q8buf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<char*>(a.q8) + slice8), (short)0, slice8_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t k8buf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<char*>(a.k8) + slice8), (short)0, slice8_bytes, 0x00020000);
        const float k_amax = a.k_amax[bh];
        const float k_r = k_amax > 0.f ? __fdiv_rn(127.f, k_amax) : 0.f;
        // Every load of the task is issued before any of its data is used: q and k rows
        // tid / 8 + 32 i of the tile (one chunk pair each), v rows 4 (tid / 64 + 4 j) + [0, 4)
        // (channels vch, vch + 1).  Rows past L read as zeros (token a.N lies past the slice).
        constexpr int kQK = kQ8Tile / (kQ8Threads / 8), kVQ = kQ8Tile / 4 / (kQ8Threads / 64);
        int nqk[kQK];
        ChunkRaw<E, kCH> wq1[kQK], wq2[kQK], wk1[kQK], wk2[kQK];
        uint32_t wv[kVQ][4][ES / 2];
#pragma unroll
        for (int i = 0; i < kQK; ++i) {
            const int p = pt * kQ8Tile + (tid >> 3) + i * (kQ8Threads / 8);
            nqk[i] = p < L ? (int)scope_token(p, s, a.sparse_k, a.mode) : a.N;
            load_pair<E>(qbuf, nqk[i] * row_bytes, rp, wq1[i], wq2[i]);
            load_pair<E>(kbuf, nqk[i] * row_bytes, rp, wk1[i], wk2[i]);
        }
#pragma unroll
        for (int j = 0; j < kVQ; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int p = pt * kQ8Tile + 4 * ((tid >> 6) + 4 * j) + r4;
                const int n = p < L ? (int)scope_token(p, s, a.sparse_k, a.mode) : a.N;
                if constexpr (ES == 2) {
                    wv[j][r4][0] = __builtin_amdgcn_raw_buffer_load_b32(vbuf, n * row_bytes + vch * ES, 0, 0);
                } else {
                    const u32x2 w2 = __builtin_amdgcn_raw_buffer_load_b64(vbuf, n * row_bytes + vch * ES, 0, 0);
                    wv[j][r4][0] = w2[0];
                    wv[j][r4][1] = w2[1];
                }
            }
        // q and k codes
#pragma unroll
        for (int i = 0; i < kQK; ++i) {
            const int n = nqk[i];
            if (n >= a.N) continue;                              // past L: uniform per group of 8 lanes
            const Pos q = grid_pos(n, a.H, a.W);
            float x1[kCH], x2[kCH];
            rotate_pair<E>(wq1[i], wq2[i], rp, tab, a.T, a.H, q, x1, x2);
            float qm = 0.f;
#pragma unroll
            for (int e = 0; e < kCH; ++e) qm = fmaxf(qm, fmaxf(fabsf(x1[e]), fabsf(x2[e])));
            qm = fmaxf(qm, __shfl_xor(qm, 1));
            qm = fmaxf(qm, __shfl_xor(qm, 2));
            qm = fmaxf(qm, __shfl_xor(qm, 4));
            const float q_r = qm > 0.f ? __fdiv_rn(127.f, qm) : 0.f;
            const int o8 = n * row8;
            __builtin_amdgcn_raw_buffer_store_b64(pack_codes(x1, q_r), q8buf, o8 + rp.c1 * kCH, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(pack_codes(x2, q_r), q8buf, o8 + rp.c2 * kCH, 0, 0);
            if (cp == 0) a.q_amax[((int64_t)b * a.N + n) * a.heads + head] = qm;
            rotate_pair<E>(wk1[i], wk2[i], rp, tab, a.T, a.H, q, x1, x2);
            __builtin_amdgcn_raw_buffer_store_b64(pack_codes(x1, k_r), k8buf, o8 + rp.c1 * kCH, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(pack_codes(x2, k_r), k8buf, o8 + rp.c2 * kCH, 0, 0);
        }
        // v codes: channels vch, vch + 1 of the row quads tid / 64 + 4 j; zero past L.  Byte r
        // of a channel's dword is row 4 q + r of the quad q (the order of the vt8 row).
        {
            float vr[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float am = a.v_amax[(int64_t)bh * kD + vch + e];
                vr[e] = am > 0.f ? __fdiv_rn(448.f, am) : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kVQ; ++j) {
                float y[4][2];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float x0, x1;
                    if constexpr (ES == 2) {
                        x0 = __uint_as_float(wv[j][r4][0] << 16);
                        x1 = __uint_as_float(wv[j][r4][0] & 0xffff0000u);
                    } else {
                        x0 = __uint_as_float(wv[j][r4][0]);
                        x1 = __uint_as_float(wv[j][r4][1]);
                    }
                    {
#pragma clang fp contract(off)
                        y[r4][0] = x0 * vr[0];
                        y[r4][1] = x1 * vr[1];
                    }
                }
                u32x2 codes;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0][e], y[1][e], 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2][e], y[3][e], w, true);
                    codes[e] = (uint32_t)w;
                }
                *reinterpret_cast<u32x2*>(vt + ((tid >> 6) + 4 * j) * kVtQuad + vch * 4) = codes;
            }
        }
        __syncthreads();
        // vt8 rows: kD channel rows of 64 bytes, four 16-byte pieces each (piece g = row quads
        // 4 g + [0, 4)); four consecutive threads write one row's 64 bytes
        unsigned char* dst = reinterpret_cast<unsigned char*>(a.vt8) + (((int64_t)bh * a.sparse_k + s) * kD) * a.Lp +
                             (int64_t)pt * kQ8Tile;
        for (int i = tid; i < kD * (kQ8Tile / 16); i += kQ8Threads) {
            const int c = i / (kQ8Tile / 16), g = i % (kQ8Tile / 16);
            u32x4 piece;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                piece[qq] = *reinterpret_cast<const uint32_t*>(vt + (4 * g + qq) * kVtQuad + 4 * c);
            *reinterpret_cast<u32x4*>(dst + (int64_t)c * a.Lp + 16 * g) = piece;
        }
        __syncthreads();
    }
}

template <typename E>
hipError_t launch_q8_t(const Q8Params& a, hipStream_t stream) {
    const size_t tab = (size_t)(a.T + a.H + a.W) * 256;
    const int nk = a.B * a.heads, nv = a.B * a.heads * kD;
    hipLaunchKernelGGL(q8_fill_kernel, dim3((nk + nv + kQ8Threads - 1) / kQ8Threads), dim3(kQ8Threads), 0, stream,
                       a.k_amax, a.v_amax, nk, nv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_stats = tab + (size_t)((kQ8Threads / 16) * kD + kQ8Threads / 64) * 4;
    const size_t lds_q = tab + (size_t)(kQ8Tile / 4) * kVtQuad;
    static_assert(SKIPARSE_MAX_GRID_SUM * 256 + ((kQ8Threads / 16) * kD + kQ8Threads / 64) * 4 <= kLdsBytes &&
                  SKIPARSE_MAX_GRID_SUM * 256 + (kQ8Tile / 4) * kVtQuad <= kLdsBytes, "the largest table fits LDS");
    // past 64 KiB of dynamic LDS (the largest grids) the kernels need the attribute
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&q8_stats_kernel<E>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_stats);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&q8_quant_kernel<E>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_q);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((q8_stats_kernel<E>), dim3((a.N + kStatTokens - 1) / kStatTokens, a.B * a.heads),
                       dim3(kQ8Threads), lds_stats, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tasks = a.B * a.heads * a.sparse_k * (a.Lp / kQ8Tile);
    hipLaunchKernelGGL((q8_quant_kernel<E>), dim3(tasks < kQ8MaxGrid ? tasks : kQ8MaxGrid), dim3(kQ8Threads),
                       lds_q, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant8(const Q8Params& a, int head_dim, int dtype, hipStream_t stream) {
    if (head_dim != kD) return hipErrorInvalidValue;
    return dtype == 0 ? launch_q8_t<BF16>(a, stream) : launch_q8_t<FP32>(a, stream);
}

int q8_scope_pitch(int L) { return (L + kQ8Tile - 1) / kQ8Tile * kQ8Tile; }

}  // namespace skiparse
