// Skiparse attention on pre-rotated q and k, and the pass that rotates them (gfx950).
//
// The fused kernel (attn_fwd.hip) rotates every K tile while staging it into LDS, and each
// of a scope's query-tile workgroups repeats that work for the same keys.  RoPE does not
// depend on the scope pattern, so here it runs once, in an HBM-bound pass, and its output
// serves every Skiparse attention over the same q and k (Single Skip and Group Skip alike):
//   rope_qk_kernel:  qr = bf16(RoPE(q) * log2(e)/sqrt(d)), kr = bf16(RoPE(k)) in token order,
//     with the same float64-evaluated cos/sin table and the same float32 arithmetic as the
//     fused kernel's staging, so qr and kr hold exactly the operands the fused kernel feeds
//     its matrix cores;
//   attn_rot_kernel: the fused kernel's workgroup shape, two-group MFMA/VALU schedule, online
//     softmax and PV product, with Q'^T read from qr straight into registers and the K tiles,
//     like the V tiles, copied from kr straight into LDS by buffer loads that write LDS.
//     The QK k-steps take head_dim in the fused kernel's order (k-step c contracts RoPE chunk
//     pair c: first-half chunk in lanes 0-31, its partner in lanes 32-63), so every product
//     and sum is the fused kernel's and the output is the same bit for bit.
// Open-Sora Plan documentation, "Skiparse Attention": RoPE on q and k at the original token
// positions, then attention within each scope.  head_dim 128, bf16, sparse_k dividing 64.
#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

using namespace attn;

namespace {

constexpr int kRD = 128;                  // head_dim
constexpr int kRCH = kRD / 16;            // elements per RoPE chunk (one 16-byte granule)
constexpr int kRWaves = 8;                // wavefronts per workgroup (2 per SIMD)
constexpr int kRThreads = 64 * kRWaves;
constexpr int kRBM = 32 * kRWaves;        // query rows per workgroup
constexpr int kRBN = 64;                  // keys per tile
constexpr int kRRow = kRD * 2;            // bytes per K / V row in LDS (bf16, unpadded)
constexpr int kRTile = kRBN * kRRow;      // bytes per K or V tile
constexpr int kRBufs = 3;                 // K tiles and V tiles in LDS
constexpr int kRKOff = 0;
constexpr int kRVOff = kRBufs * kRTile;
constexpr int kRLds = 2 * kRBufs * kRTile;

constexpr int kRopeWaves = 4;             // rotation pass: wavefronts (tokens) per workgroup

// K tile row r: logical granule g of the row is stored at granule g ^ krswz(r).  The QK operand
// reads fetch one granule of 16 consecutive rows per 16 lanes, which then fall on 16 distinct
// granule positions, i.e. all 64 banks; the loads into LDS write whole 1 KiB pieces.
__device__ __forceinline__ int krswz(int r) { return r & 15; }

// Chunk of head_dim that lane half hf contributes to QK k-step ks (RoPE chunk pair ks)
__device__ __forceinline__ int qk_chunk(int ks, int hf) {
    const RopePair rp = rope_pair(ks);
    return hf ? rp.c2 : rp.c1;
}

}  // namespace

// ---- the rotation pass: one wavefront per token, one RoPE chunk per lane ----
// A wavefront rotates every head row of one token of q and of k.  Lane l owns RoPE chunk
// c = l % 16 of head rows l / 16, l / 16 + 4, ..., so the eight (cos, sin) pairs it needs are
// the same for all its rows.  The token's 64 pairs (16 on the t axis, 24 on h, 24 on w) are
// evaluated one per lane, with the float64 expressions of the attention kernels' table
// (build_banked_rope_table) rounded to float32, so the rotated rows hold exactly the operands
// the fused kernel computes; that evaluation runs while the first loads are in flight.  The
// rotate-half partner chunk of c lies 2 (t axis) or 3 (h, w) chunks away in the same head
// row, i.e. in a lane of the same group of 16, and is fetched with a cross-lane permute.
// Loads are nontemporal (read once); stores are ordinary write-back stores, since the
// attention that follows reads q' and k' right away.  One-shot grid: one wavefront per
// token, no loop over tokens.
__global__ void __launch_bounds__(64 * kRopeWaves) rope_qk_kernel(RopeQkParams a) {
    __shared__ __attribute__((aligned(16))) float2 pairs[kRopeWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tok = (int64_t)blockIdx.x * kRopeWaves + wave;     // b * N + n
    if (tok >= (int64_t)a.B * a.N) return;
    const int n = (int)(tok % a.N);
    const int c = lane & 15;
    // the chunk pair of chunk c (rope_pair order: t pairs 0-1, h pairs 2-4, w pairs 5-7)
    const int cp = c < 4 ? (c & 1) : (c < 10 ? 2 + (c - 4) % 3 : 5 + (c - 10) % 3);
    const RopePair rp = rope_pair(cp);
    const bool first = c == rp.c1;
    const int partner = (lane & ~15) + (first ? rp.c2 : rp.c1);
    const int base = (rp.axis == 0 ? 0 : (rp.axis == 1 ? 16 : 40)) + rp.jchunk * kRCH;
    const int64_t row0 = tok * a.heads * kRRow;         // byte offset of the token's first head row
    const int hrows = (a.heads + 3) / 4;                // head rows per lane
    constexpr int kU = 6;                               // head rows per lane per round
    u32x4 w[2][kU];
    auto load_round = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int which = 0; which < 2; ++which)
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int h = min(4 * (i0 + u) + (lane >> 4), a.heads - 1);
                const char* in = reinterpret_cast<const char*>(which == 0 ? a.q : a.k) + row0 + h * kRRow + c * 16;
                w[which][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in));
            }
    };
    load_round(0);
    {
        // pair `lane` of the token: t axis pairs 0-15 (d_t = 32), h 16-39, w 40-63 (d = 48)
        const int axis = lane < 16 ? 0 : (lane < 40 ? 1 : 2);
        const int j = lane - (axis == 0 ? 0 : (axis == 1 ? 16 : 40));
        const int pos = axis == 0 ? n / (a.H * a.W) : (axis == 1 ? (n / a.W) % a.H : n % a.W);
        const double da = axis == 0 ? (double)(kRD / 4) : (double)(3 * kRD / 8);
        const double inv_freq = pow(10000.0, -2.0 * (double)j / da);
        const double theta = (double)pos * inv_freq;
        double sn, cs;
        sincos(theta, &sn, &cs);
        pairs[wave][lane] = make_float2((float)cs, (float)sn);
    }
    __builtin_amdgcn_wave_barrier();
    f32x4 cs[kRCH / 2];
#pragma unroll
    for (int i = 0; i < kRCH / 2; ++i) cs[i] = *reinterpret_cast<const f32x4*>(&pairs[wave][base + 2 * i]);
    for (int i0 = 0; i0 < hrows; i0 += kU) {
        if (i0 > 0) load_round(i0);
#pragma unroll
        for (int which = 0; which < 2; ++which)
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int h = 4 * (i0 + u) + (lane >> 4);
                u32x4 oth;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    oth[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(partner * 4, (int)w[which][u][q]);
                ChunkRaw<BF16, kRCH> r1, r2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    r1.w[q] = first ? w[which][u][q] : oth[q];
                    r2.w[q] = first ? oth[q] : w[which][u][q];
                }
                float x1[kRCH], x2[kRCH];
                raw_to_f32(r1, x1);
                raw_to_f32(r2, x2);
                rope_rotate_cs<kRCH>(x1, x2, cs);
                if (which == 0) {
#pragma unroll
                    for (int e = 0; e < kRCH; ++e) {
                        x1[e] *= a.scale_log2;
                        x2[e] *= a.scale_log2;
                    }
                }
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = first ? pack_bf16x2(x1[2 * q], x1[2 * q + 1]) : pack_bf16x2(x2[2 * q], x2[2 * q + 1]);
                char* out = reinterpret_cast<char*>(which == 0 ? a.qr : a.kr) + row0 + h * kRRow + c * 16;
                if (i0 + u < hrows && h < a.heads) *reinterpret_cast<u32x4*>(out) = o;
            }
    }
}

// ---- attention on qr, kr, v ----
// LSE: also write each row's log2-sum-exp for the backward (a separate instantiation, so the
// plain forward carries none of its code).
template <bool LSE>
__global__ void __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(kRThreads / 256, kRThreads / 256)))
attn_rot_kernel(AttnParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int KS = kRD / 16;   // 16-deep k-steps of Q K^T
    constexpr int DB = kRD / 32;   // 32-row blocks of O^T
    constexpr int KB = kRBN / 32;  // 32-key blocks of S^T
    constexpr int KK = kRBN / 16;  // 16-deep k-steps of P V
    constexpr int G = kRD / 8;     // 16-byte granules per row

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
    const int row_bytes = a.heads * kRRow;                 // bytes per token
    // buffer descriptors over this (batch, head) slice; tokens >= N lie past its end
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * kRRow;
    const int slice_bytes = a.N * row_bytes - head * kRRow;
    const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.q) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t obuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<char*>(a.out) + slice), (short)0, slice_bytes, 0x00020000);

    // ---- Q'^T of the wave's 32 query rows, straight from qr into registers ----
    bf16x8 qreg[KS];
    {
        const int p = qt * kRBM + wave * 32 + l32;
        const int off = (int)scope_token(p, s, k_, a.mode) * row_bytes;   // past the slice: zeros
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qbuf, off + qk_chunk(ks, hf) * 16, 0, 0));
    }

    // ---- tile loads into LDS: each wave moves two 1 KiB pieces (4 rows each) of every K tile
    // and two of every V tile; in a piece, lane l fills LDS granule l of the piece with the
    // granule of row l / G that the row's swizzle puts there ----
    constexpr int kOps = kRBN * G / 64 / kRWaves;   // pieces per wave per tile
    static_assert(kOps == 2, "two pieces per wave and tile");
    const int tile_dn = kRBN * a.sparse_k;          // token advance per tile (sparse_k | 64)
    int koff[kOps], voff[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        const int r = (wave * kOps + i) * (64 / G) + lane / G;
        const int tok = (int)scope_token(r, s, k_, a.mode);
        koff[i] = tok * row_bytes + ((lane % G) ^ krswz(r)) * 16;
        voff[i] = tok * row_bytes + ((lane % G) ^ vswz<kRD>(r)) * 16;
    }
    // each call moves the next tile (the cursors advance one tile per call)
    auto load_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kOps; ++i) {
            buffer_load_to_lds16(kbuf, lds + kRKOff + buf * kRTile + (wave * kOps + i) * 1024, koff[i]);
            koff[i] += tile_dn * row_bytes;
        }
    };
    auto load_v = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kOps; ++i) {
            buffer_load_to_lds16(vbuf, lds + kRVOff + buf * kRTile + (wave * kOps + i) * 1024, voff[i]);
            voff[i] += tile_dn * row_bytes;
        }
    };

    // QK operand reads: row 32 kb + l32, logical granule qk_chunk(ks, hf)
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = l32 * kRRow + ((qk_chunk(ks, hf) ^ krswz(l32)) << 4);
    // PV operand reads with ds_read_b64_tr_b16, as in the fused kernel: within each group of
    // 16 lanes, lane 4t + j points at 4 consecutive d of key row t and receives element j of
    // each of those 4 keys; lanes 0-31 read keys {0-3, 8-11} and lanes 32-63 keys {4-7, 12-15}
    // of every 16-key step (the order of P^T in the accumulator layout).
    const int tr_i = lane & 15;
    const int tr_row = (tr_i >> 2) + 4 * (lane >> 5);
    const int tr_gran = 2 * ((lane >> 4) & 1) + ((tr_i & 3) >> 1);
    const int tr_byte = (tr_i & 1) * 8;
    auto v_rd = [&](int h, int db) __attribute__((always_inline)) {
        const int r = 8 * h + tr_row;
        return r * kRRow + (((4 * db + tr_gran) ^ vswz<kRD>(r)) * 16) + tr_byte;
    };

    // ---- accumulators and softmax state: scores arrive as S' = s*log2(e)/sqrt(d) - m_ref ----
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
    float m_ref = 0.f, l_part = 0.f;
    f32x16 s_init;
#pragma unroll
    for (int x = 0; x < 16; ++x) s_init[x] = 0.f;
    const int nt = (a.L + kRBN - 1) / kRBN;
    f32x16 sacc[KB];
    bf16x8 pb[KK];

    // S'^T = K Q'^T onto -m_ref, 16 MFMAs in (ks, kb) order.  Every MFMA operand below comes
    // through a 2-deep register ring (read one step ahead): measured 2.7 % faster than 4-deep
    // and 1 % faster than 3-deep here (fewer LDS reads in flight per wave, 212 VGPRs), while
    // one step ahead is too little (19 % slower).
    constexpr int kRing = 2;
    auto qk = [&](int buf) __attribute__((always_inline)) {
        const char* kcur = lds + kRKOff + buf * kRTile;
        constexpr int NST = KS * KB;
        auto kop = [&](int st) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8*>(kcur + k_rd[st / KB] + (st % KB) * 32 * kRRow);
        };
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = s_init;
        bf16x8 ka[kRing];
#pragma unroll
        for (int st = 0; st < kRing - 1; ++st) ka[st] = kop(st);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (st + kRing - 1 < NST) ka[(st + kRing - 1) % kRing] = kop(st + kRing - 1);
            sacc[st % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[st % kRing], qreg[st / KB], sacc[st % KB], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kRing - 1, 0);
#pragma unroll
        for (int i = 0; i < NST - (kRing - 1); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kRing - 1, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // online softmax of tile j (softmax_tile, as in the fused kernel)
    auto softmax = [&](int j) __attribute__((always_inline)) {
        softmax_tile<DB, true>(sacc, o, pb, s_init, m_ref, l_part, j == 0,
                         j == nt - 1 && (a.L % kRBN) != 0, a.L - j * kRBN, hf);
    };

    // O^T += V^T P^T, V^T operands by transpose reads through the ring
    auto pv = [&](int buf) __attribute__((always_inline)) {
        const char* vcur = lds + kRVOff + buf * kRTile;
        constexpr int NST = KK * DB;
        auto vop = [&](int st) __attribute__((always_inline)) {
            const int kk = st / DB, db = st % DB;
            const i16x4 lo = ds_read_tr16(vcur + (16 * kk) * kRRow + v_rd(0, db));
            const i16x4 hi = ds_read_tr16(vcur + (16 * kk) * kRRow + v_rd(1, db));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8, v);
        };
        bf16x8 va[kRing];
#pragma unroll
        for (int st = 0; st < kRing - 1; ++st) va[st] = vop(st);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (st + kRing - 1 < NST) va[(st + kRing - 1) % kRing] = vop(st + kRing - 1);
            o[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[st % kRing], pb[st / DB], o[st % DB], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (kRing - 1), 0);
#pragma unroll
        for (int i = 0; i < NST - (kRing - 1); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kRing - 1, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- schedule ----
    // Waves 0-3 (group 0) and 4-7 (group 1) alternate between an MFMA block and a VALU block,
    // one phase apart, a workgroup barrier closing every phase.  Phases ph = 1, 2, ...; group
    // g runs MFMA block m = (ph - 1 - g) / 2 when ph + g is odd (PV(m-1) if m >= 1, QK(m) if
    // m < nt) and VALU block m = (ph - 2 + g) / 2 when ph + g is even: its pieces of V tile m+1
    // and K tile m+2 requested into LDS, softmax(m) (g = 0) or softmax(m-1) (g = 1), then a
    // wait for the requests of the wave's previous VALU block.
    // K tile m sits in K buffer m % 3 and V tile m in V buffer m % 3.  K tile m+2 is requested
    // in phases 2m+1 / 2m+2, after QK(m-1), the last reader of its buffer, ended (phases 2m-1
    // and 2m), and has landed after phase 2m+4, before QK(m+2) in phase 2m+5.  V tile m+1 is
    // requested in the same phases, after PV(m-2) ended (phases 2m-1, 2m), and has landed
    // before PV(m+1) in phase 2m+5.
    const int grp = wave >= kRWaves / 2 ? 1 : 0;
    // Wave-uniform: the wave has a query row inside the scope.  A wave of the scope's ragged
    // last q tile whose 32 rows all lie past its end skips its products and softmax but still
    // moves its share of every K/V tile and joins every barrier (k = 8 on the 24x22x40 grid:
    // 5 of the last tile's 8 waves, 2 % of the kernel's time).
    const bool busy = qt * kRBM + wave * 32 < a.L;
    load_k(0);
    if (nt > 1) load_k(1);
    load_v(0);
    wait_vm_loads();
    __syncthreads();
    auto opaque = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
    // PV(m-1) and QK(m) as one sequence of 32 MFMAs whose operands come through one ring, so
    // the first QK operands are read while the last PV products run
    auto mfma_both = [&](int vb, int kbuf) __attribute__((always_inline)) {
        const char* vcur = lds + kRVOff + vb * kRTile;
        const char* kcur = lds + kRKOff + kbuf * kRTile;
        constexpr int NPV = KK * DB, NQK = KS * KB, NST = NPV + NQK;
        auto op = [&](int st) __attribute__((always_inline)) {
            if (st < NPV) {
                const int kk = st / DB, db = st % DB;
                const i16x4 lo = ds_read_tr16(vcur + (16 * kk) * kRRow + v_rd(0, db));
                const i16x4 hi = ds_read_tr16(vcur + (16 * kk) * kRRow + v_rd(1, db));
                const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                return __builtin_bit_cast(bf16x8, v);
            }
            const int t = st - NPV;
            return *reinterpret_cast<const bf16x8*>(kcur + k_rd[t / KB] + (t % KB) * 32 * kRRow);
        };
        bf16x8 ra[kRing];
#pragma unroll
        for (int st = 0; st < kRing - 1; ++st) ra[st] = op(st);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if (st + kRing - 1 < NST) ra[(st + kRing - 1) % kRing] = op(st + kRing - 1);
            if (st < NPV) {
                o[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st % kRing], pb[st / DB], o[st % DB], 0, 0, 0);
            } else {
                const int t = st - NPV;
                sacc[t % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st % kRing], qreg[t / KB], t < KB ? s_init : sacc[t % KB], 0, 0, 0);
            }
        }
        constexpr int kPro = (kRing - 1) * 2;
        __builtin_amdgcn_sched_group_barrier(0x100, kPro, 0);
#pragma unroll
        for (int i = 0; i < NPV - (kRing - 1); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int i = NPV - (kRing - 1); i < NST - (kRing - 1); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kRing - 1, 0);
        __builtin_amdgcn_s_setprio(0);
    };
    auto valu_block = [&](int m, int sm) __attribute__((always_inline)) {
        const bool lv = m + 1 < nt, lk = m + 2 < nt;
        if (lv) load_v(opaque((m + 1) % 3));
        if (lk) load_k(opaque((m + 2) % 3));
        if (busy && sm >= 0 && sm < nt) softmax(sm);
        if (lk) wait_vm_loads_but<2 * kOps>();   // this block's requests may stay in flight
        else if (lv) wait_vm_loads_but<kOps>();
        else wait_vm_loads();
    };
    // The first and last MFMA blocks (QK(0) alone, PV(nt-1) alone) are peeled off the loops.
    if (grp == 0) {
        if (busy) qk(0);
        __syncthreads();
        valu_block(0, 0);
        __syncthreads();
        for (int m = 1; m < nt; ++m) {
            if (busy) mfma_both(opaque((m - 1) % 3), opaque(m % 3));
            __syncthreads();
            valu_block(m, m);
            __syncthreads();
        }
        if (busy) pv(opaque((nt - 1) % 3));
        __syncthreads();
        valu_block(nt, nt);
        __syncthreads();
    } else {
        valu_block(0, -1);
        __syncthreads();
        if (busy) qk(0);
        __syncthreads();
        for (int m = 1; m < nt; ++m) {
            valu_block(m, m - 1);
            __syncthreads();
            if (busy) mfma_both(opaque((m - 1) % 3), opaque(m % 3));
            __syncthreads();
        }
        valu_block(nt, nt - 1);
        __syncthreads();
        if (busy) pv(opaque((nt - 1) % 3));
        __syncthreads();
    }

    // ---- epilogue: normalise and scatter rows back to their tokens ----
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / l_tot;
        const int p = qt * kRBM + wave * 32 + l32;
        const int n_tok = (int)scope_token(p, s, k_, a.mode);
        const int off = n_tok * row_bytes;   // past the slice when p >= L
        if (LSE && hf == 0 && p < a.L)
            a.lse[((int64_t)b * a.heads + head) * a.N + n_tok] = m_ref + log2f(l_tot);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hf;
                const float y0 = o[db][4 * g] * inv, y1 = o[db][4 * g + 1] * inv;
                const float y2 = o[db][4 * g + 2] * inv, y3 = o[db][4 * g + 3] * inv;
                const u32x2 v2 = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                __builtin_amdgcn_raw_buffer_store_b64(v2, obuf, off + d0 * 2, 0, 0);
            }
    }
}

hipError_t launch_rope_qk(const RopeQkParams& a, hipStream_t stream) {
    const int64_t tokens = (int64_t)a.B * a.N;
    const int64_t blocks = (tokens + kRopeWaves - 1) / kRopeWaves;
    hipLaunchKernelGGL(rope_qk_kernel, dim3((unsigned)blocks), dim3(64 * kRopeWaves), 0, stream, a);
    return hipGetLastError();
}

template <bool LSE>
static hipError_t launch_attn_rot_l(const AttnParams& a, hipStream_t stream) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_rot_kernel<LSE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kRLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_rot_kernel<LSE>, dim3(a.num_work), dim3(kRThreads), kRLds, stream, a);
    return hipGetLastError();
}

hipError_t launch_attn_rot(const AttnParams& a, hipStream_t stream) {
    return a.lse != nullptr ? launch_attn_rot_l<true>(a, stream) : launch_attn_rot_l<false>(a, stream);
}

}  // namespace skiparse
