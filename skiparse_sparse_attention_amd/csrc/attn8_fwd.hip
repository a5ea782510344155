// 8-bit Skiparse attention forward for gfx950 (CDNA4).
//
// Wan 2.1 report, section 4.4.3 "Quantization" (paragraph "8-Bit FlashAttention"): scores from
// Int8 operands, S = Q K^T on the int8 matrix cores, and O = P V from FP8 (E4M3) operands, with
// each key block's PV products reduced on the matrix cores and the running sum over blocks
// kept in float32 (on CDNA4 the FP8 matrix instruction accumulates in float32 itself, so the
// block products go straight into the float32 O accumulator, rescaled when the reference
// maximum moves).  The operands come from quant8.hip: q8 and k8 (int8, original token order,
// after RoPE), q_amax (one per query row), k_amax (one per batch and head), vt8 (E4M3 values,
// transposed per scope) and v_amax (one per channel).
//
// Per (batch, head, scope), for query row i and key j of the scope:
//   z_ij = (q8_i . k8_j) * (q_amax_i / 127) * (k_amax / 127) * log2(e) / sqrt(d)
//   M_i  = ceil(max_j z_ij)          P_ij = 2^(z_ij - M_i + 8)  in (0, 256]
//   O_i  = (sum_j E4M3(P_ij) * V~_j) * (v_amax / 448) / sum_j P_ij
// The kernel keeps an integer running reference m_i: the ceiling of the first tile's maximum,
// moved to the ceiling of a later tile's maximum only when that maximum exceeds m_i by more
// than 0.8, so every weight stays at or below 2^8.8 < 448 (the largest E4M3 value).  A move
// multiplies O and the row sum by 2^(m_old - m_new), an exact power of two, so every weight is
// quantised on the same grid (up to powers of two) as against the final M_i, E4M3's subnormal
// range aside.  (Moving on every rise of the ceiling rescaled about a third of the tiles of
// random inputs; the 0.8 margin skips part of those rescales: 2.3 % less kernel time on the
// 24x22x40 workload.)
//
// Tiling and schedule follow the bf16 kernel (attn_fwd.hip): one workgroup = 8 wavefronts =
// 256 query rows of one scope, 32 per wavefront, two groups of four wavefronts alternating
// between an MFMA block and a VALU block one phase apart.  Differences:
//   * Q'^T is the B operand of v_mfma_i32_32x32x32_i8, 16 int8 per lane per k-step, loaded
//     straight from q8 into registers; the K tile (64 rows of 128 int8) is the A operand in
//     LDS.  K and V^T tiles reach LDS through registers: each wave fetches its 16 bytes per lane
//     of both tiles one VALU block ahead and writes them to LDS with ds_write_b128 (the loads
//     that write LDS directly measured 6-9 % slower here, against 2-4 % faster in the bf16
//     rotated kernel, whose VALU blocks are shorter);
//   * the key rows of the two 32-row S^T blocks of a tile are permuted so that lane l of the
//     accumulators holds keys 32 (l / 32) + [0, 32) of the tile; those 32 weights, converted
//     to E4M3 in register order, are the B operand of v_mfma_scale_f32_32x32x64_f8f6f4 (unit
//     scales), and the A operand, V^T, is read from the transposed vt8 tile as 32 consecutive
//     keys of one channel per lane, two 16-byte LDS reads;
//   * both tiles are XOR-swizzled per row so every LDS operand read is bank-conflict-free.
#include <type_traits>

#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

using namespace attn;

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kD8 = 128;                  // head_dim of the 8-bit path
constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kBM8 = 32 * kWaves8;        // query rows per workgroup
constexpr int kBN8 = 64;                  // keys per tile
constexpr int kKTile8 = kBN8 * kD8;       // K tile bytes (64 rows of 128 int8)
constexpr int kVTile8 = kD8 * kBN8;       // V^T tile bytes (128 channel rows of 64 E4M3)
constexpr int kBufs8 = 3;
constexpr int kKOff8 = 0;
constexpr int kVOff8 = kBufs8 * kKTile8;
constexpr int kLds8 = kBufs8 * (kKTile8 + kVTile8);
constexpr float kPHeadroom = 8.0f;        // largest weight 2^8
constexpr float kScaleLog2 = (float)(1.4426950408889634 / 11.313708498984761);   // log2(e) / sqrt(128)

// K tile row r (a key of the tile): granule g of the 128-byte row is stored at g ^ kswz(r).
// The QK operand reads of a 16-lane group touch the keys {16 b + 0..7, 32 + 16 b + 0..7} at
// one logical granule; kswz spreads them over all 16 (row parity, granule) bank groups.
__device__ __forceinline__ int kswz(int r) { return ((r >> 1) & 3) | ((r >> 3) & 4); }
// V^T tile row c (a channel): granule g of the 64-byte row is stored at g ^ vtswz(c); the 16
// rows read by a 16-lane group then cover every (row mod 4, granule) bank group.
__device__ __forceinline__ int vtswz(int c) { return (c >> 2) & 3; }

}  // namespace

__global__ void __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn8_fwd_kernel(Attn8Params a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int KSQ = kD8 / 32;   // 32-deep k-steps of Q K^T
    constexpr int DB = kD8 / 32;    // 32-channel blocks of O^T
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;

    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = work % a.q_tiles;
    const int sc = work / a.q_tiles;
    const int s = sc % a.sparse_k;
    const int bh = sc / a.sparse_k;
    const int head = bh % a.heads;
    const int b = bh / a.heads;
    const int64_t k_ = a.sparse_k;
    const int row8 = a.heads * kD8;                               // bytes per token of q8 / k8
    const int64_t slice8 = ((int64_t)b * a.N * a.heads + head) * kD8;
    const int slice8_bytes = a.N * row8 - head * kD8;
    const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.q8) + slice8), (short)0, slice8_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k8) + slice8), (short)0, slice8_bytes, 0x00020000);
    const int64_t vslice = ((int64_t)bh * a.sparse_k + s) * kD8 * a.Lp;
    const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.vt8) + vslice), (short)0, kD8 * a.Lp, 0x00020000);
    // q_amax of this (batch, head): element n at byte 4 * (n * heads); n >= N reads 0
    const __amdgpu_buffer_rsrc_t qabuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q_amax + (int64_t)b * a.N * a.heads + head), (short)0, (a.N * a.heads - head) * 4, 0x00020000);
    const int ob = a.out_bytes;
    const int64_t oslice = ((int64_t)b * a.N * a.heads + head) * kD8 * ob;
    const int oslice_bytes = a.N * a.heads * kD8 * ob - head * kD8 * ob;
    const __amdgpu_buffer_rsrc_t obuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<char*>(a.out) + oslice), (short)0, oslice_bytes, 0x00020000);

    // ---- Q'^T operand and the per-query score scale ----
    const int p_q = qt * kBM8 + wave * 32 + l32;
    const int n_q = (int)scope_token(p_q, s, k_, a.mode);      // >= N past the scope end
    i32x4 qreg[KSQ];
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks)
        qreg[ks] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(qbuf, n_q * row8 + 32 * ks + 16 * hf, 0, 0));
    const float q_amax = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(qabuf, n_q * a.heads * 4, 0, 0));
    // z = acc * cq in base-2 units of the scaled scores
    const float cq = (q_amax * (1.0f / 127.0f)) * (a.k_amax[bh] * (1.0f / 127.0f)) * kScaleLog2;

    // ---- tile loads: each wave moves 1 KiB of the K tile and 1 KiB of the V^T tile ----
    // K piece w: rows 8w + lane/8, LDS granule lane%8 holds logical granule (lane%8) ^ kswz(row)
    const int k_row = wave * 8 + (lane >> 3);
    const int k_gran = (lane & 7) ^ kswz(k_row);
    // V^T piece w: channel rows 16w + lane/4, LDS granule lane%4 holds (lane%4) ^ vtswz(c)
    const int v_row = wave * 16 + (lane >> 2);
    const int v_gran = (lane & 3) ^ vtswz(v_row);
    const int tile_dn = kBN8 * a.sparse_k;   // token advance per tile (sparse_k divides 64)
    int koff = (int)scope_token(k_row, s, k_, a.mode) * row8 + 16 * k_gran;
    int voff = v_row * a.Lp + 16 * v_gran;
    i32x4 kst, vst;   // this wave's 16-byte pieces of the next K and V^T tiles, in flight
    auto fetch_k = [&]() __attribute__((always_inline)) {
        kst = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(kbuf, koff, 0, 0));
        koff += tile_dn * row8;
    };
    auto fetch_v = [&]() __attribute__((always_inline)) {
        vst = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(vbuf, voff, 0, 0));
        voff += kBN8;
    };
    auto put_k = [&](int buf) __attribute__((always_inline)) {
        *reinterpret_cast<i32x4*>(lds + kKOff8 + buf * kKTile8 + wave * 1024 + lane * 16) = kst;
    };
    auto put_v = [&](int buf) __attribute__((always_inline)) {
        *reinterpret_cast<i32x4*>(lds + kVOff8 + buf * kVTile8 + wave * 1024 + lane * 16) = vst;
    };

    // ---- LDS operand addresses ----
    // QK A operand for S^T block kb: lane row rho = l32 holds key pi(kb, rho) =
    // 32 (rho/4 % 2) + 16 kb + 4 (rho / 8) + rho % 4, so that the accumulator rows 8j + 4h + r
    // of lane half h are the tile's keys 32 h + 16 kb + 4 j + r.
    const int rho_h = (l32 >> 2) & 1, rho_j = l32 >> 3, rho_r = l32 & 3;
    const int key0 = 32 * rho_h + 4 * rho_j + rho_r;            // + 16 kb
    const int kf = kswz(key0);                                  // same for key0 + 16
    int k_rd[KSQ];
#pragma unroll
    for (int ks = 0; ks < KSQ; ++ks) k_rd[ks] = key0 * kD8 + (((2 * ks + hf) ^ kf) << 4);
    // PV A operand for O^T block db: channel 32 db + l32, keys 32 hf + [0, 32): granules 2 hf, 2 hf + 1
    const int vf = vtswz(l32);
    const int v_rd0 = l32 * kBN8 + (((2 * hf) ^ vf) << 4);
    const int v_rd1 = l32 * kBN8 + (((2 * hf + 1) ^ vf) << 4);

    // ---- state ----
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
    float m_run = 0.f, l_part = 0.f;
    const int nt = (a.L + kBN8 - 1) / kBN8;
    i32x16 sacc[2];
    i32x8 pbytes;

    auto qk = [&](int buf) __attribute__((always_inline)) {
        const char* kt = lds + kKOff8 + buf * kKTile8;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[kb][x] = 0;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KSQ; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const i32x4 ka = *reinterpret_cast<const i32x4*>(kt + k_rd[ks] + kb * 16 * kD8);
                sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qreg[ks], sacc[kb], 0, 0, 0);
            }
        __builtin_amdgcn_s_setprio(0);
    };

    // `masked`: the last tile of the scope, whose keys past the end of the scope are excluded
    // from the maximum and weighted 0.  Only the peeled last iteration of each schedule loop
    // instantiates it, so the loop body carries none of the masking.
    auto softmax = [&](int j, auto masked) __attribute__((always_inline)) {
        constexpr bool ragged = decltype(masked)::value;
        const int valid = a.L - j * kBN8;
        if constexpr (ragged) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    if (32 * hf + 16 * kb + 4 * (x >> 2) + (x & 3) >= valid) sacc[kb][x] = INT32_MIN;
        }
        int mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = max(mx, sacc[kb][x]);
        const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)mx, (unsigned)mx, false, false);
        mx = max((int)sw[0], (int)sw[1]);
        const float zt = (float)mx * cq;
        const float mt = __builtin_ceilf(zt);
        const bool grow = zt > m_run + 0.8f;
        if (j == 0) {
            m_run = mt;
        } else if (__ballot(grow) != 0ull) {
            const float alpha = grow ? __builtin_ldexpf(1.0f, (int)(m_run - mt)) : 1.0f;
            m_run = grow ? mt : m_run;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) o[db][x] *= alpha;
        }
        const float bias = kPHeadroom - m_run;
        float lsum[2] = {l_part, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = __builtin_fmaf((float)sacc[kb][4 * g + r], cq, bias);
                    if constexpr (ragged)
                        if (32 * hf + 16 * kb + 4 * g + r >= valid) t = -__builtin_inff();
                    p[r] = __builtin_amdgcn_exp2f(t);
                    // the second chain starts at its first weight (0 + p is p)
                    if (kb == 0 && g == 0 && r == 1) lsum[1] = p[r];
                    else lsum[r & 1] += p[r];
                }
                // weights of keys 32 hf + 16 kb + 4 g + [0, 4): bytes 16 kb + 4 g + [0, 4) of the operand;
                // both halves of the register are rewritten, so the old value is passed through
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pbytes[4 * kb + g], false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                pbytes[4 * kb + g] = w;
            }
        l_part = lsum[0] + lsum[1];
    };

    auto pv = [&](int buf) __attribute__((always_inline)) {
        const char* vt = lds + kVOff8 + buf * kVTile8;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(vt + db * 32 * kBN8 + v_rd0);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(vt + db * 32 * kBN8 + v_rd1);
            const i32x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            // format 0 = E4M3 for both operands; scale exponents 127 = 2^0
            o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pbytes, o[db], 0, 0, 0, 127, 0, 127);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- schedule (phases as in attn_fwd.hip) ----
    // Group 0 runs MFMA block m in phase 2m and VALU block m in phase 2m+1, group 1 runs VALU
    // block m in phase 2m and MFMA block m in phase 2m+1.  MFMA block m: PV(m-1) if m >= 1,
    // QK(m) if m < nt.  VALU block m: softmax(m) (group 0) or softmax(m-1) (group 1), a wait for
    // the fetches of the wave's previous VALU block, V^T tile m and K tile m+1 written to their
    // buffers, then V^T tile m+1 and K tile m+2 fetched into registers.  K tile m+1 goes to K
    // buffer (m+1) % 3 in phases 2m, 2m+1, after its last reader QK(m-2) (phases 2m-4, 2m-3),
    // and is read by QK(m+1) from phase 2m+2 on; V^T tile m goes to V buffer m % 3 after PV(m-3)
    // (MFMA block m-2) and is read by PV(m) in MFMA block m+1.  The prologue writes K tile 0
    // and fetches V^T tile 0 and K tile 1.
    const int grp = wave >= kWaves8 / 2 ? 1 : 0;
    fetch_k();
    wait_vm_loads();
    put_k(0);
    fetch_v();
    if (nt > 1) fetch_k();
    __syncthreads();
    auto opaque = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
    auto mfma_block = [&](int m) __attribute__((always_inline)) {
        if (m >= 1) pv(opaque((m - 1) % 3));
        if (m < nt) qk(opaque(m % 3));
    };
    // VALU block m: softmax, then V^T tile m and K tile m+1 (fetched in block m-1) written to
    // their buffers, then V^T tile m+1 and K tile m+2 fetched
    auto valu_block = [&](int m, int sm, auto masked) __attribute__((always_inline)) {
        if (sm >= 0 && sm < nt) softmax(sm, masked);
        wait_vm_loads();
        if (m < nt) put_v(opaque(m % 3));
        if (m + 1 < nt) put_k(opaque((m + 1) % 3));
        if (m + 1 < nt) fetch_v();
        if (m + 2 < nt) fetch_k();
    };
    // softmax(nt - 1), the only one that may need masking, runs in group 0's VALU block
    // m = nt - 1 and in group 1's VALU block m = nt: those iterations are peeled
    const std::false_type plain;
    const std::true_type last;
    if (grp == 0) {
        for (int m = 0; m < nt - 1; ++m) {
            mfma_block(m);
            __syncthreads();
            valu_block(m, m, plain);
            __syncthreads();
        }
        mfma_block(nt - 1);
        __syncthreads();
        valu_block(nt - 1, nt - 1, last);
        __syncthreads();
        mfma_block(nt);
        __syncthreads();
        valu_block(nt, nt, plain);   // no loads and no softmax left: the final wait only
        __syncthreads();
    } else {
        for (int m = 0; m < nt; ++m) {
            valu_block(m, m - 1, plain);
            __syncthreads();
            mfma_block(m);
            __syncthreads();
        }
        valu_block(nt, nt - 1, last);
        __syncthreads();
        mfma_block(nt);
        __syncthreads();
    }

    // ---- epilogue: O / l * v_amax / 448, scattered back to the query's token row ----
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = (1.0f / 448.0f) / l_tot;
        const float* va = a.v_amax + (int64_t)bh * kD8;
        const int off = n_q * a.heads * kD8 * ob;   // past the slice when the row is past the scope
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = db * 32 + 8 * g + 4 * hf;
                const f32x4 vs = *reinterpret_cast<const f32x4*>(va + c0);
                const float y0 = o[db][4 * g] * (vs[0] * inv), y1 = o[db][4 * g + 1] * (vs[1] * inv);
                const float y2 = o[db][4 * g + 2] * (vs[2] * inv), y3 = o[db][4 * g + 3] * (vs[3] * inv);
                if (ob == 2) {
                    const u32x2 v2 = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                    __builtin_amdgcn_raw_buffer_store_b64(v2, obuf, off + c0 * 2, 0, 0);
                } else {
                    const u32x4 v4 = {__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3)};
                    __builtin_amdgcn_raw_buffer_store_b128(v4, obuf, off + c0 * 4, 0, 0);
                }
            }
    }
}

hipError_t launch_attn8(const Attn8Params& a, hipStream_t stream) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn8_fwd_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds8);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn8_fwd_kernel, dim3(a.num_work), dim3(kThreads8), kLds8, stream, a);
    return hipGetLastError();
}

int attn8_block_rows() { return kBM8; }

}  // namespace skiparse
