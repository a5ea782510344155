// Fused Skiparse attention forward for gfx950 (CDNA4).
//
// Computes, for every (batch b, head, scope s), softmax(Q_s K_s^T / sqrt(d)) V_s
// where Q_s, K_s, V_s are the rows of scope s (Open-Sora Plan documentation,
// "Skiparse Attention": Single Skip / Group Skip), with 3D RoPE applied to the
// q and k rows at their original grid positions, and writes each output row
// back to its original token index (the page's reverse_sparse).  Nothing
// rearranged is ever written to memory:
//   * the gather happens in the tile loads: row p of scope s is token
//     n(s, p), whose (batch, token, head) row is read directly;
//   * RoPE is applied while staging q and k tiles into LDS, from a cos/sin
//     table each workgroup builds in LDS;
//   * the epilogue stores row p straight to token n(s, p).
//
// Tiling (one workgroup = 8 wavefronts = 256 query rows of one scope; two wavefronts per
// SIMD):
//   * each wavefront owns 32 query rows and keeps Q^T for them in registers as the B
//     operand of v_mfma_f32_32x32x16_bf16;
//   * K tiles of 64 keys are staged (rotated, bf16, row-major) in LDS and are the A operand,
//     so the scores come out transposed: S^T = K Q^T.  In the 32x32 accumulator layout a
//     lane then owns one query column and 16 of its keys per 32-key block, so row sums and
//     maxima are in-lane reductions plus one swap with the lane 32 away;
//   * P^T (bf16) is fed to O^T += V^T P^T straight from the accumulator registers as the B
//     operand.  The MFMA contracts over whatever key order the operand slots carry; V is
//     copied row-major into LDS by buffer loads that write LDS directly, and its V^T
//     operands are read with the LDS transpose read ds_read_b64_tr_b16, whose per-lane
//     addresses pick the keys in exactly the slot order in which P^T's accumulator layout
//     holds them;
//   * online softmax in fp32 on exp2: the scale log2(e)/sqrt(d) is folded into q before its
//     bf16 rounding and the QK MFMAs accumulate onto -m_ref, so the scores arrive already
//     shifted and each weight costs one v_exp_f32.  The tile softmax (softmax_tile, shared
//     with the rotated kernel) sums the unrounded weights in fp32; the reference m_ref is set
//     from the first tile's row maxima and afterwards moved only when some lane's 32 weights
//     of a tile sum to more than 2^8 (the result is identical up to rounding, since the same
//     reference scales numerator and denominator), which skips almost every rescale of the
//     O^T accumulator and every tile maximum on the common path;
//   * the two wavefronts of each SIMD belong to different groups (waves 0-3, waves 4-7), and
//     the groups alternate between an MFMA block (PV of the previous tile, QK of the current
//     one) and a VALU block (softmax, RoPE staging of the next K tile, load requests), one
//     phase apart with a workgroup barrier per phase, so one wave's MFMAs run beside the
//     other's vector work;
//   * LDS layouts are bank-conflict-free for every access: padded Q/K rows, XOR-swizzled V
//     rows, and a RoPE table with one row per axis position at axis-dependent offsets;
//   * all global traffic uses buffer instructions with 32-bit offsets into the
//     (batch, head) slice; rows past the end of a scope have token indices >= N, i.e.
//     offsets past the slice, which the hardware range check turns into zero loads and
//     dropped stores;
//   * workgroup ids are remapped so the q tiles of one scope run on the same XCD and share
//     its L2 copy of the scope's K and V.
#include <type_traits>

#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

namespace {

constexpr int kWaves = 8;                 // wavefronts per workgroup (2 per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;          // query rows per workgroup (32 per wavefront)
constexpr int kBN = 64;                   // keys per tile

template <int D>
struct Lds {
    static constexpr int kRowPitch = D * 2 + 16;          // Q / K rows (bf16) + one pad granule
    static constexpr int kVPitch = D * 2;                 // V rows (bf16), granules swizzled
    static constexpr int kKTile = kBN * kRowPitch;
    static constexpr int kVTile = kBN * kVPitch;
    static constexpr int kKBufs = 2;                      // K tiles in LDS (see the schedule)
    static constexpr int kVBufs = 3;                      // V tiles in LDS
    static constexpr int kKOff = 0;
    static constexpr int kVOff = kKBufs * kKTile;
    static constexpr int kTiles = kKBufs * kKTile + kVBufs * kVTile;
    static constexpr int kQBytes = kBM * kRowPitch;       // Q staging, aliases the tiles
    static constexpr int kTabOff = kTiles > kQBytes ? kTiles : kQBytes;
    static constexpr int kTabRow = 256;                   // bytes per RoPE table row
};

}  // namespace

using namespace attn;

// KDIV: sparse_k divides kBN, so row p + kBN of a scope is token n(p) + kBN*k in both modes
// and the load cursors advance by a constant.  LSE: also write each row's log2-sum-exp (a
// separate instantiation, so the plain forward carries none of its code).
template <int D, typename E, bool KDIV, bool LSE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kThreads / 256, kThreads / 256)))
attn_fwd_kernel(AttnParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef Lds<D> L;
    constexpr int CH = D / 16;   // elements per RoPE chunk
    constexpr int CB = CH * 2;   // bytes per RoPE chunk in LDS (bf16)
    constexpr int KS = D / 16;   // 16-deep k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    constexpr int KB = kBN / 32; // 32-key blocks of S^T
    constexpr int KK = kBN / 16; // 16-deep k-steps of P V
    constexpr int ES = E::kBytes;
    char* tab = lds + L::kTabOff;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int l32 = lane & 31, hf = lane >> 5;

    // ---- which (batch, head, scope, q tile) this workgroup computes ----
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = work % a.q_tiles;
    const int sc = work / a.q_tiles;
    const int s = sc % a.sparse_k;
    const int bh = sc / a.sparse_k;
    const int head = bh % a.heads;
    const int b = bh / a.heads;
    const int64_t k_ = a.sparse_k;
    const int row_bytes = a.heads * D * ES;                 // bytes per token
    // Buffer descriptors over this (batch, head) slice.  Offsets are token*row_bytes +
    // byte-in-head-row; every token >= N lies past the slice (reads 0, store dropped).
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * ES;
    const int slice_bytes = a.N * row_bytes - head * D * ES;
    const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.q) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.k) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.v) + slice), (short)0, slice_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t obuf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<char*>(a.out) + slice), (short)0, slice_bytes, 0x00020000);
    const int HW = a.H * a.W;

    build_banked_rope_table<D>(tab, a.T, a.H, a.W, a.phi_mul);

    // This thread's RoPE chunk pair (same for its Q and K staging tasks) and the byte
    // offsets of its table entries: tab_base + pos * 256 (+ 16 * phi on the w axis).
    const int cp = tid & 7;
    const RopePair rp = rope_pair(cp);
    const int tab_base = (rp.axis == 0 ? 0
                          : rp.axis == 1 ? a.T * 256 + RopeBank<D>::kOffH * 16
                                         : (a.T + a.H) * 256 + RopeBank<D>::kOffW * 16) +
                         rp.jchunk * CH * 8;
    const int tab_phi_mul = rp.axis == 2 ? a.phi_mul : 0;
    // the CH (cos, sin) pairs of this thread's chunk pair at grid position q, as CH/2 16-byte reads
    auto load_tab = [&](const Pos& q, f32x4 (&cs)[CH / 2]) __attribute__((always_inline)) {
        // t can exceed T-1 only on rows past the end of the scope, whose data is zero
        const int pos = rp.axis == 0 ? min(q.t, a.T - 1) : (rp.axis == 1 ? q.h : q.w);
        const char* row = tab + tab_base + pos * 256 + rope_phi(pos, tab_phi_mul) * 16;
#pragma unroll
        for (int i = 0; i < CH / 2; ++i) cs[i] = *reinterpret_cast<const f32x4*>(row + 16 * i);
    };
    auto pos_of = [&](int nn) __attribute__((always_inline)) {
        Pos q;
        q.t = nn / HW; q.h = (nn / a.W) % a.H; q.w = nn % a.W;
        return q;
    };
    // byte offsets, inside a Q/K row, of the chunks of this thread's pair (slots 2 cp, 2 cp + 1)
    const int c1_off = 2 * cp * CB, c2_off = (2 * cp + 1) * CB;

    // ---- stage the Q tile (rotated) into LDS, then into registers ----
    {
        const int p0 = qt * kBM;
        __syncthreads();  // table ready
#pragma unroll 2
        for (int it = 0; it < kBM * 8 / kThreads; ++it) {
            const int r = (tid >> 3) + it * (kThreads / 8);
            const int n = (int)scope_token(p0 + r, s, k_, a.mode);   // >= N past the scope end
            const int off = n * row_bytes;
            ChunkRaw<E, CH> r1, r2;
            buffer_load_dwords(qbuf, off + rp.c1 * CH * ES, r1.w);
            buffer_load_dwords(qbuf, off + rp.c2 * CH * ES, r2.w);
            float x1[CH], x2[CH];
            raw_to_f32(r1, x1);
            raw_to_f32(r2, x2);
            f32x4 cs[CH / 2];
            load_tab(pos_of(n), cs);
            rope_rotate_cs<CH>(x1, x2, cs);
            // fold the softmax scale log2(e)/sqrt(d) into q: scores come out in log2 units
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                x1[e] *= a.scale_log2;
                x2[e] *= a.scale_log2;
            }
            store_rotated_chunks<CH>(lds + r * L::kRowPitch + c1_off, lds + r * L::kRowPitch + c2_off, x1, x2);
        }
    }
    __syncthreads();
    bf16x8 qreg[KS];
    {
        const int qr = wave * 32 + l32;
        const char* qrow = lds + qr * L::kRowPitch;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + hf) * 16);
    }
    __syncthreads();  // the Q area is reused by the K/V buffers below

    // ---- per-thread staging assignment ----
    // K: one (key row, RoPE chunk pair) task per thread.
    // V: rows are copied unchanged in 1 KiB pieces (kVRows whole rows): in piece i, lane l
    //    moves granule l % G of row i*kVRows + l / G into LDS position l, loading for it the
    //    granule that the row swizzle puts there.  Each wave moves kVOps pieces per tile.
    static_assert(kBN * 8 == kThreads, "one K staging task per thread");
    constexpr int G = D / 8;                      // 16-byte bf16 granules per row
    constexpr int kVRows = 64 / G;                // rows per 1 KiB piece
    constexpr int kVOps = kBN / kVRows / kWaves;  // pieces per wave per tile
    static_assert(kVOps * kVRows * kWaves == kBN, "whole V tile in 1 KiB pieces");
    const int krow = tid >> 3;
    int vrow[kVOps], vgran[kVOps];
#pragma unroll
    for (int i = 0; i < kVOps; ++i) {
        vrow[i] = (wave * kVOps + i) * kVRows + lane / G;
        vgran[i] = (lane % G) ^ vswz<D>(vrow[i]);
    }

    // loop-invariant LDS addresses (the buffer base is added per tile)
    const int k_wr1 = krow * L::kRowPitch + c1_off;
    const int k_wr2 = krow * L::kRowPitch + c2_off;
    // PV operand reads with ds_read_b64_tr_b16.  Within each group of 16 lanes, lane
    // i = 4t + q points at 4 consecutive d of key row t; the instruction then hands lane j
    // the value at d0 + j of each of those 4 keys.  Lanes 0-31 need keys {0-3, 8-11} and
    // lanes 32-63 keys {4-7, 12-15} of every 16-key step (the order in which the 32x32
    // accumulator layout holds P^T), d0 = 16 * ((lane / 16) % 2) within a 32-row block.
    // Row 16 kk + 8 h + tr_row, granule 4 db + tr_gran, byte tr_byte within the granule.
    const int tr_i = lane & 15;
    const int tr_row = (tr_i >> 2) + 4 * (lane >> 5);
    const int tr_gran = 2 * ((lane >> 4) & 1) + ((tr_i & 3) >> 1);
    const int tr_byte = (tr_i & 1) * 8;
    auto v_rd = [&](int h, int db) __attribute__((always_inline)) {
        const int r = 8 * h + tr_row;   // the row modulo 16, which is all vswz looks at
        return r * L::kVPitch + (((4 * db + tr_gran) ^ vswz<D>(r)) * 16) + tr_byte;
    };

    // Global offsets of the rows to be loaded next (the load cursor runs two tiles ahead
    // of the compute) and grid position of the K row to be staged next.
    int koff1, koff2, voff[kVOps];
    Pos kpos;
    const int tile_dn = kBN * a.sparse_k;     // token advance per tile when k | kBN
    const int dt = tile_dn / HW, rem = tile_dn % HW;
    const int dh = rem / a.W, dw = rem % a.W;
    auto set_k_rows = [&](int p0) __attribute__((always_inline)) {
        const int kn = (int)scope_token(p0 + krow, s, k_, a.mode);
        koff1 = kn * row_bytes + rp.c1 * CH * ES;
        koff2 = kn * row_bytes + rp.c2 * CH * ES;
    };
    auto set_v_rows = [&](int p0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kVOps; ++i)
            voff[i] = (int)scope_token(p0 + vrow[i], s, k_, a.mode) * row_bytes + vgran[i] * 8 * ES;
    };
    auto advance_k_rows = [&](int tile) __attribute__((always_inline)) {   // to tile `tile`, from tile - 1
        if constexpr (KDIV) {
            koff1 += tile_dn * row_bytes;
            koff2 += tile_dn * row_bytes;
        } else {
            set_k_rows(tile * kBN);
        }
    };
    auto advance_v_rows = [&](int tile) __attribute__((always_inline)) {
        if constexpr (KDIV) {
#pragma unroll
            for (int i = 0; i < kVOps; ++i) voff[i] += tile_dn * row_bytes;
        } else {
            set_v_rows(tile * kBN);
        }
    };
    auto advance_stage_pos = [&](int tile) __attribute__((always_inline)) {   // to tile `tile`, from tile - 1
        if constexpr (KDIV) {
            int w = kpos.w + dw, c = w >= a.W;
            kpos.w = w - (c ? a.W : 0);
            int h = kpos.h + dh + c;
            c = h >= a.H;
            kpos.h = h - (c ? a.H : 0);
            kpos.t += dt + c;
        } else {
            kpos = pos_of((int)scope_token(tile * kBN + krow, s, k_, a.mode));
        }
    };
    set_k_rows(0);
    set_v_rows(0);
    kpos = pos_of((int)scope_token(krow, s, k_, a.mode));

    // K rows: loaded into registers two phases before they are rotated and staged.
    // V rows: bf16 goes straight from memory into the LDS tile (buffer loads to LDS); fp32 is
    // loaded through registers and rounded to bf16.
    ChunkRaw<E, CH> kraw[2];
    auto load_k = [&]() __attribute__((always_inline)) {
        buffer_load_dwords(kbuf, koff1, kraw[0].w);
        buffer_load_dwords(kbuf, koff2, kraw[1].w);
    };
    auto load_v = [&](int vb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kVOps; ++i) {
            char* dst = lds + L::kVOff + vb * L::kVTile + (wave * kVOps + i) * 1024;
            if constexpr (ES == 2) {
                buffer_load_to_lds16(vbuf, dst, voff[i]);
            } else {
                uint32_t w[4];
                buffer_load_8_as_bf16x2<E>(vbuf, voff[i], w);
                *reinterpret_cast<u32x4*>(dst + lane * 16) = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    };
    // vector memory instructions one staging block issues (the V loads to LDS, then the K loads)
    constexpr int kKLoadOps = 2 * (CH * ES >= 32 ? 2 : 1);
    constexpr int kVmOps = (ES == 2 ? kVOps : 0) + kKLoadOps;

    // table entries for the K row to be staged next, read at the start of the staging block
    f32x4 kcs[CH / 2];
    auto stage_k = [&](int kb) __attribute__((always_inline)) {
        char* kdst = lds + L::kKOff + kb * L::kKTile;
        float x1[CH], x2[CH];
        raw_to_f32(kraw[0], x1);
        raw_to_f32(kraw[1], x2);
        rope_rotate_cs<CH>(x1, x2, kcs);
        store_rotated_chunks<CH>(kdst + k_wr1, kdst + k_wr2, x1, x2);
    };

    // ---- accumulators and softmax state ----
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
    // Softmax reference: scores are kept as S' = s*log2(e)/sqrt(d) - m_ref, with m_ref the
    // running reference maximum (log2 units).  The QK MFMAs start from an accumulator that
    // holds -m_ref in every slot, so they produce S' directly.
    float m_ref = 0.f, l_part = 0.f;
    f32x16 s_init;
#pragma unroll
    for (int x = 0; x < 16; ++x) s_init[x] = 0.f;
    const int nt = (a.L + kBN - 1) / kBN;

    // ---- the four blocks of work per key tile ----
    f32x16 sacc[KB];     // S'^T of the tile being processed
    bf16x8 pb[KK];       // its bf16 weights, the B operand of P V

    // S'^T = K Q'^T onto -m_ref.  The 16 MFMAs run in (ks, kb) order; their K operands
    // come from a 4-deep register ring, read 3 steps ahead.
    constexpr int kRing = 4;
    auto qk = [&](int buf) __attribute__((always_inline)) {
        const char* kcur = lds + L::kKOff + buf * L::kKTile;
        constexpr int NST = KS * KB;
        // The lane's K read offset is recomputed here rather than held across the loop: at 256
        // VGPRs the compiler otherwise spilled it and reloaded it at the start of every QK
        // block, behind a wait for all of the wave's outstanding loads (the tile prefetch).
        int lid = (int)threadIdx.x;
        asm volatile("" : "+v"(lid));
        const int k_rd_t = (lid & 31) * L::kRowPitch + ((lid >> 5) & 1) * 16;   // + kb*32 rows + ks*32 bytes
        auto kop = [&](int st) __attribute__((always_inline)) {
            return *reinterpret_cast<const bf16x8*>(kcur + k_rd_t + (st % KB) * 32 * L::kRowPitch + (st / KB) * 32);
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

    // online softmax of tile j (softmax_tile: weights P = exp2(S'), row sums, lazy reference)
    auto softmax = [&](int j) __attribute__((always_inline)) {
        softmax_tile<DB>(sacc, o, pb, s_init, m_ref, l_part, j == 0,
                         j == nt - 1 && (a.L % kBN) != 0, a.L - j * kBN, hf);
    };

    // O^T += V^T P^T; the V^T operands come transposed out of the row-major V tile, two
    // transpose reads per operand, through a 4-deep register ring read 3 steps ahead.
    auto pv = [&](int buf) __attribute__((always_inline)) {
        const char* vcur = lds + L::kVOff + buf * L::kVTile;
        constexpr int NST = KK * DB;
        auto vop = [&](int st) __attribute__((always_inline)) {
            const int kk = st / DB, db = st % DB;
            const i16x4 lo = ds_read_tr16(vcur + (16 * kk) * L::kVPitch + v_rd(0, db));
            const i16x4 hi = ds_read_tr16(vcur + (16 * kk) * L::kVPitch + v_rd(1, db));
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
    // Waves 0-3 (group 0, one per SIMD) and waves 4-7 (group 1) alternate between an MFMA
    // block and a VALU block, one phase apart, with a workgroup barrier closing every phase,
    // so on each SIMD one wave's MFMAs run beside the other wave's vector work.  Phase
    // numbers ph = 1, 2, ...; group g runs in phase ph
    //   MFMA block (ph + g odd), m = (ph - 1 - g) / 2:   PV(m-1) if m >= 1, QK(m) if m < nt;
    //   VALU block (ph + g even), m = (ph - 2 + g) / 2:  softmax(m) (g = 0) or softmax(m-1)
    //     (g = 1); the group's half of the rows of K tile m+1 rotated and staged; its half of
    //     V tile m+1 requested into LDS; its K rows of tile m+2 requested into registers.
    // K tile m lives in K buffer m % 2 and V tile m in V buffer m % 3.  K tile m+1 is staged
    // in phases 2m+1 and 2m+2, after the last reads of K tile m-1 (QK(m-1) in phases 2m-1 and
    // 2m) and before the first read (QK(m+1) in phase 2m+3).  V tile m+1 is requested in
    // phases 2m+1 and 2m+2, after the last reads of V tile m-2 (PV(m-2) in phases 2m-1 and
    // 2m); each VALU block ends by waiting until the loads of the wave's previous VALU block
    // have landed, so V tile m+1 is complete after phase 2m+4, before PV(m+1) in phase 2m+5.
    // P(m) stays in registers from softmax(m) to PV(m) in the group's next MFMA block.
    const int grp = wave >= kWaves / 2 ? 1 : 0;   // wave-uniform
    // prologue: K tile 0 staged by every wave, V tile 0 in LDS, the K rows of tile 1 requested
    load_v(0);
    load_k();
    load_tab(kpos, kcs);
    stage_k(0);
    if (nt > 1) {
        advance_k_rows(1);
        load_k();
    }
    wait_vm_loads();
    __syncthreads();

    // Buffer indices pass through readfirstlane, which keeps the compiler from turning every
    // LDS address of the loop into an induction variable of its own.
    auto opaque = [](int x) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(x); };
    auto mfma_block = [&](int m) __attribute__((always_inline)) {
        if (m >= 1) pv(opaque((m - 1) % 3));
        if (m < nt) qk(opaque(m & 1));
    };
    auto valu_block = [&](int m, int sm) __attribute__((always_inline)) {
        if (m + 1 < nt) {
            advance_v_rows(m + 1);
            load_v(opaque((m + 1) % 3));
        }
        if (sm >= 0 && sm < nt) softmax(sm);
        if (m + 1 < nt) {
            advance_stage_pos(m + 1);
            load_tab(kpos, kcs);
            stage_k(opaque((m + 1) & 1));
        }
        if (m + 2 < nt) {
            advance_k_rows(m + 2);
            load_k();
            wait_vm_loads_but<kVmOps>();   // this block's loads may stay in flight
        } else {
            wait_vm_loads();
        }
    };
    // One loop per group, so that only P (group 0) or only S (group 1) is carried around
    // each loop's back edge.
    if (grp == 0) {
        for (int m = 0; m <= nt; ++m) {
            mfma_block(m);       // phase 2m+1
            __syncthreads();
            valu_block(m, m);    // phase 2m+2
            __syncthreads();
        }
    } else {
        for (int m = 0; m <= nt; ++m) {
            valu_block(m, m - 1);   // phase 2m+1
            __syncthreads();
            mfma_block(m);          // phase 2m+2
            __syncthreads();
        }
    }

    // ---- epilogue: normalise and scatter rows back to their tokens ----
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / l_tot;
        const int p = qt * kBM + wave * 32 + l32;
        const int n_tok = (int)scope_token(p, s, k_, a.mode);
        const int off = n_tok * row_bytes;   // past the slice when p >= L
        // log2-sum-exp of the row's scaled scores, for the backward pass
        if (LSE && hf == 0 && p < a.L)
            a.lse[((int64_t)b * a.heads + head) * a.N + n_tok] = m_ref + log2f(l_tot);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * hf;
                const float y0 = o[db][4 * g] * inv, y1 = o[db][4 * g + 1] * inv;
                const float y2 = o[db][4 * g + 2] * inv, y3 = o[db][4 * g + 3] * inv;
                if constexpr (ES == 2) {
                    const u32x2 v2 = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                    __builtin_amdgcn_raw_buffer_store_b64(v2, obuf, off + d0 * 2, 0, 0);
                } else {
                    const u32x4 v4 = {__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3)};
                    __builtin_amdgcn_raw_buffer_store_b128(v4, obuf, off + d0 * 4, 0, 0);
                }
            }
    }
}

template <int D, typename E, bool KDIV, bool LSE>
static hipError_t launch_attn_k(const AttnParams& a, hipStream_t stream) {
    typedef Lds<D> L;
    static_assert(L::kTabOff + SKIPARSE_MAX_GRID_SUM * L::kTabRow <= kLdsBytes, "the largest table fits LDS");
    const size_t lds = (size_t)L::kTabOff + (size_t)(a.T + a.H + a.W) * L::kTabRow;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<D, E, KDIV, LSE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, E, KDIV, LSE>), dim3(a.num_work), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <int D, typename E, bool LSE>
static hipError_t launch_attn_l(const AttnParams& a, hipStream_t stream) {
    return a.k_divides_bn ? launch_attn_k<D, E, true, LSE>(a, stream) : launch_attn_k<D, E, false, LSE>(a, stream);
}

template <int D, typename E>
static hipError_t launch_attn_t(const AttnParams& a, hipStream_t stream) {
    return a.lse != nullptr ? launch_attn_l<D, E, true>(a, stream) : launch_attn_l<D, E, false>(a, stream);
}

hipError_t launch_attn(const AttnParams& a, int head_dim, int dtype, hipStream_t stream) {
    if (head_dim == 128) return dtype == 0 ? launch_attn_t<128, BF16>(a, stream) : launch_attn_t<128, FP32>(a, stream);
    return dtype == 0 ? launch_attn_t<64, BF16>(a, stream) : launch_attn_t<64, FP32>(a, stream);
}

int attn_block_rows() { return kBM; }
int attn_tile_keys() { return kBN; }

}  // namespace skiparse
