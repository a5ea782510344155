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
// through LDS.
#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

using namespace attn;

namespace {

constexpr int kQ8Threads = 256;        // 4 wavefronts
constexpr int kQ8Tile = 64;            // scope positions per quantisation task
constexpr int kStatTokens = 512;       // tokens per statistics workgroup
constexpr int kQ8MaxGrid = 1024;       // quantisation workgroups (each builds the table once)

// Pair i of a head row (i < D/2): the RoPE axis, its frequency index j and the offsets of the
// two rotate-half elements (axis chunks t, h, w of D/4, 3D/8, 3D/8 elements).
template <int D>
struct PairSlot {
    int axis, j, e1, e2;
    __device__ __forceinline__ explicit PairSlot(int i) {
        constexpr int ht = D / 8, hh = 3 * D / 16;
        if (i < ht) {
            axis = 0; j = i; e1 = i; e2 = i + ht;
        } else if (i < ht + hh) {
            axis = 1; j = i - ht; e1 = D / 4 + j; e2 = e1 + hh;
        } else {
            axis = 2; j = i - ht - hh; e1 = 5 * D / 8 + j; e2 = e1 + hh;
        }
    }
};

// x1' = x1 c - x2 s, x2' = x2 c + x1 s with every product and sum rounded to float32
__device__ __forceinline__ void rotate_rn(float x1, float x2, float2 cs, float& y1, float& y2) {
#pragma clang fp contract(off)
    y1 = x1 * cs.x - x2 * cs.y;
    y2 = x2 * cs.x + x1 * cs.y;
}

template <typename E>
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (E::kBytes == 2)
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
    else
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// int8 code of x * r (r = 127 / amax), both float32 operations rounded to nearest even
__device__ __forceinline__ int int8_code(float x, float r) {
#pragma clang fp contract(off)
    const float y = __builtin_rintf(x * r);
    return (int)fminf(fmaxf(y, -127.f), 127.f);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// Grid position of token n and the table offset of pair `ps` at it.
template <int D>
__device__ __forceinline__ const float2* pair_cs(const char* tab, const Q8Params& a, const PairSlot<D>& ps, int n) {
    const int HW = a.H * a.W;
    const int pos = ps.axis == 0 ? n / HW : (ps.axis == 1 ? (n / a.W) % a.H : n % a.W);
    return reinterpret_cast<const float2*>(tab + rope_tab_offset<D>(a.T, a.H, ps.axis, pos, ps.j, 0));
}

__global__ void __launch_bounds__(kQ8Threads) q8_fill_kernel(float* k_amax, float* v_amax, int nk, int nv) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nk + nv; i += gridDim.x * blockDim.x) {
        if (i < nk) k_amax[i] = 0.f;
        else v_amax[i - nk] = 0.f;
    }
}

// Statistics: workgroup (token chunk, batch * heads + head).  Lane l of a row group handles
// RoPE pair l of k and channels 2l, 2l + 1 of v; a wavefront covers 128 / D token rows per
// step.
template <int D, typename E>
__global__ void __launch_bounds__(kQ8Threads) q8_stats_kernel(Q8Params a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int LPR = D / 2;              // lanes per token row
    constexpr int RPW = 64 / LPR;           // token rows per wavefront step
    constexpr int ES = E::kBytes;
    char* tab = lds;
    float* red = reinterpret_cast<float*>(lds + (a.T + a.H + a.W) * 256);   // [4 waves][RPW][D + 1]
    const int bh = blockIdx.y, b = bh / a.heads, head = bh % a.heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LPR, li = lane % LPR;
    const int row_bytes = a.heads * D * ES;
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * ES;
    const int slice_bytes = a.N * row_bytes - head * D * ES;
    const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
    build_banked_rope_table<D>(tab, a.T, a.H, a.W, 0);
    __syncthreads();
    const PairSlot<D> ps(li);
    float km = 0.f, vm0 = 0.f, vm1 = 0.f;
    const int n0 = blockIdx.x * kStatTokens;
    const int n1 = min(n0 + kStatTokens, a.N);
    for (int n = n0 + wave * RPW + sub; n < n1; n += 4 * RPW) {
        const int off = n * row_bytes;
        float y1, y2;
        rotate_rn(load_elem<E>(kbuf, off + ps.e1 * ES), load_elem<E>(kbuf, off + ps.e2 * ES),
                  *pair_cs<D>(tab, a, ps, n), y1, y2);
        km = fmaxf(km, fmaxf(fabsf(y1), fabsf(y2)));
        vm0 = fmaxf(vm0, fabsf(load_elem<E>(vbuf, off + 2 * li * ES)));
        vm1 = fmaxf(vm1, fabsf(load_elem<E>(vbuf, off + (2 * li + 1) * ES)));
    }
    km = wave_max(km);
    float* wr = red + (wave * RPW + sub) * (D + 1);
    wr[2 * li] = vm0;
    wr[2 * li + 1] = vm1;
    if (lane == 0) wr[D] = km;
    __syncthreads();
    for (int c = tid; c <= D; c += kQ8Threads) {
        float m = 0.f;
        for (int r = 0; r < 4 * RPW; ++r) m = fmaxf(m, red[r * (D + 1) + c]);
        unsigned* dst = c < D ? reinterpret_cast<unsigned*>(a.v_amax) + (int64_t)bh * D + c
                              : reinterpret_cast<unsigned*>(a.k_amax) + bh;
        atomicMax(dst, __float_as_uint(m));
    }
}

// Quantisation: task (batch, head, scope, tile of 64 scope positions).  Each wavefront takes
// 16 positions: q and k rows by RoPE pair per lane (codes stored straight to their original
// token rows), v by channel pair per lane into a transposed LDS tile, which the workgroup
// then writes as 64-byte rows of vt8.
template <int D, typename E>
__global__ void __launch_bounds__(kQ8Threads) q8_quant_kernel(Q8Params a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int LPR = D / 2;
    constexpr int RPW = 64 / LPR;
    constexpr int ES = E::kBytes;
    constexpr int kVtPitch = kQ8Tile + 4;                       // bytes per transposed LDS row
    char* tab = lds;
    unsigned char* vt = reinterpret_cast<unsigned char*>(lds + (a.T + a.H + a.W) * 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LPR, li = lane % LPR;
    const int row_bytes = a.heads * D * ES;
    const int row8 = a.heads * D;                               // bytes per token of q8 / k8
    const int L = a.N / a.sparse_k;
    const int tiles = a.Lp / kQ8Tile;
    const int tasks = a.B * a.heads * a.sparse_k * tiles;
    build_banked_rope_table<D>(tab, a.T, a.H, a.W, 0);
    __syncthreads();
    const PairSlot<D> ps(li);
    for (int task = blockIdx.x; task < tasks; task += gridDim.x) {
        const int pt = task % tiles;
        const int s = (task / tiles) % a.sparse_k;
        const int bh = task / (tiles * a.sparse_k);
        const int b = bh / a.heads, head = bh % a.heads;
        const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * ES;
        const int slice_bytes = a.N * row_bytes - head * D * ES;
        const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.q) + slice), (short)0, slice_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
        const int64_t slice8 = ((int64_t)b * a.N * a.heads + head) * D;
        const int slice8_bytes = a.N * row8 - head * D;
        const __amdgpu_buffer_rsrc_t q8buf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<char*>(a.q8) + slice8), (short)0, slice8_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t k8buf = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<char*>(a.k8) + slice8), (short)0, slice8_bytes, 0x00020000);
        const float k_amax = a.k_amax[bh];
        const float k_r = k_amax > 0.f ? __fdiv_rn(127.f, k_amax) : 0.f;
        const float* va = a.v_amax + (int64_t)bh * D;
        const float vam0 = va[2 * li], vam1 = va[2 * li + 1];
        const float v_r0 = vam0 > 0.f ? __fdiv_rn(448.f, vam0) : 0.f;
        const float v_r1 = vam1 > 0.f ? __fdiv_rn(448.f, vam1) : 0.f;
        for (int rr = wave * RPW + sub; rr < kQ8Tile; rr += 4 * RPW) {
            const int p = pt * kQ8Tile + rr;
            const int n = p < L ? (int)scope_token(p, s, a.sparse_k, a.mode) : a.N;   // a.N: reads 0
            const int off = n * row_bytes;
            const float2 cs = n < a.N ? *pair_cs<D>(tab, a, ps, n) : make_float2(1.f, 0.f);
            // q: per-row amax across the LPR lanes of the row
            float q1, q2;
            rotate_rn(load_elem<E>(qbuf, off + ps.e1 * ES), load_elem<E>(qbuf, off + ps.e2 * ES), cs, q1, q2);
            float qm = fmaxf(fabsf(q1), fabsf(q2));
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) qm = fmaxf(qm, __shfl_xor(qm, m));
            const float q_r = qm > 0.f ? __fdiv_rn(127.f, qm) : 0.f;
            float k1, k2;
            rotate_rn(load_elem<E>(kbuf, off + ps.e1 * ES), load_elem<E>(kbuf, off + ps.e2 * ES), cs, k1, k2);
            if (n < a.N) {
                const int o8 = n * row8;
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)int8_code(q1, q_r), q8buf, o8 + ps.e1, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)int8_code(q2, q_r), q8buf, o8 + ps.e2, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)int8_code(k1, k_r), k8buf, o8 + ps.e1, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)int8_code(k2, k_r), k8buf, o8 + ps.e2, 0, 0);
                if (li == 0) a.q_amax[((int64_t)b * a.N + n) * a.heads + head] = qm;
            }
            // v: E4M3 codes of channels 2 li, 2 li + 1 into the transposed tile (zero past L)
            const float x0 = load_elem<E>(vbuf, off + 2 * li * ES), x1 = load_elem<E>(vbuf, off + (2 * li + 1) * ES);
            float y0, y1;
            {
#pragma clang fp contract(off)
                y0 = x0 * v_r0;
                y1 = x1 * v_r1;
            }
            const unsigned pk = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
            vt[(2 * li) * kVtPitch + rr] = (unsigned char)(pk & 0xff);
            vt[(2 * li + 1) * kVtPitch + rr] = (unsigned char)((pk >> 8) & 0xff);
        }
        __syncthreads();
        // vt8 rows: D channel rows of 64 bytes, 16 bytes per thread step
        unsigned char* dst = reinterpret_cast<unsigned char*>(a.vt8) + (((int64_t)bh * a.sparse_k + s) * D) * a.Lp +
                             (int64_t)pt * kQ8Tile;
        for (int i = tid; i < D * (kQ8Tile / 16); i += kQ8Threads) {
            const int c = i / (kQ8Tile / 16), g = i % (kQ8Tile / 16);
            const unsigned char* src = vt + c * kVtPitch + 16 * g;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)src[4 * e] | ((uint32_t)src[4 * e + 1] << 8) | ((uint32_t)src[4 * e + 2] << 16) |
                       ((uint32_t)src[4 * e + 3] << 24);
            *reinterpret_cast<u32x4*>(dst + (int64_t)c * a.Lp + 16 * g) = w;
        }
        __syncthreads();
    }
}

template <int D, typename E>
hipError_t launch_q8_t(const Q8Params& a, hipStream_t stream) {
    const size_t tab = (size_t)(a.T + a.H + a.W) * 256;
    const int nk = a.B * a.heads, nv = a.B * a.heads * D;
    hipLaunchKernelGGL(q8_fill_kernel, dim3((nk + nv + kQ8Threads - 1) / kQ8Threads), dim3(kQ8Threads), 0, stream,
                       a.k_amax, a.v_amax, nk, nv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_stats = tab + (size_t)4 * (64 / (D / 2)) * (D + 1) * 4;
    hipLaunchKernelGGL((q8_stats_kernel<D, E>), dim3((a.N + kStatTokens - 1) / kStatTokens, a.B * a.heads),
                       dim3(kQ8Threads), lds_stats, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tasks = a.B * a.heads * a.sparse_k * (a.Lp / kQ8Tile);
    const size_t lds_q = tab + (size_t)D * (kQ8Tile + 4);
    hipLaunchKernelGGL((q8_quant_kernel<D, E>), dim3(tasks < kQ8MaxGrid ? tasks : kQ8MaxGrid), dim3(kQ8Threads),
                       lds_q, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant8(const Q8Params& a, int head_dim, int dtype, hipStream_t stream) {
    if (head_dim == 128) return dtype == 0 ? launch_q8_t<128, BF16>(a, stream) : launch_q8_t<128, FP32>(a, stream);
    return dtype == 0 ? launch_q8_t<64, BF16>(a, stream) : launch_q8_t<64, FP32>(a, stream);
}

int q8_scope_pitch(int L) { return (L + kQ8Tile - 1) / kQ8Tile * kQ8Tile; }

}  // namespace skiparse
