// Fused Skiparse attention backward for gfx950 (CDNA4).
//
// Gradients through the forward of attn_fwd.hip (3D RoPE on q and k at the original grid
// positions, Single/Group Skip scopes, softmax attention per scope, scatter back to the
// original tokens).  Given dO (the loss gradient of the output, original token order), the
// forward output O and the forward's per-row log2-sum-exp, compute dQ, dK, dV in the original
// token order.  Per (batch, head, scope), with Z = c q' k'^T (c = 1/sqrt(d); q', k' rotated)
// and P = softmax(Z) row-wise, the chain rule gives
//   D   = rowsum(dO * O)                (equal to rowsum(P * dP))
//   dV  = P^T dO
//   dP  = dO V^T,  dZ = P * (dP - D)
//   dq' = c dZ k',  dk' = c dZ^T q'
// and dq, dk are dq', dk' turned back by the transposed RoPE rotation (each rotate-half pair
// by -theta).  Wan 2.1 report, section 4.3.1, prices this backward at twice the forward.
//
// Two kernels, both recomputing P from the scores and the saved log2-sum-exp:
//   attn_bwd_dq_kernel: one workgroup per (batch, head, scope, 256-query tile), 8 wavefronts
//     of 32 queries.  It computes D of its queries (and stores it for the second kernel),
//     then streams the scope's 64-key K/V tiles: S^T = K Q'^T onto -LSE, P^T = exp2(S^T),
//     dP^T = V dO^T, dZ^T = P^T * (dP^T - D), dQ'^T += K^T dZ^T, the K^T operands read from
//     the row-major K tile with the LDS transpose read.
//   attn_bwd_dkdv_kernel: one workgroup per (batch, head, scope, 128-key tile), 8 wavefronts,
//     two on each 32-key group; streams the scope's 64-query tiles: S = Q' K'^T onto -LSE, P,
//     dP = dO V^T, dZ, dV^T += dO^T P, dK^T += Q'^T dZ, the dO^T and Q'^T operands again from
//     transpose reads.
// Rows are gathered through the scope map on load (q and k rotated while staged into LDS
// from the banked RoPE table), the transposed rotation is applied in registers in the
// epilogue, and every gradient row is written straight to its original token.  Keys past the
// end of a scope start at -inf (weight exactly 0); queries past the end carry an infinite
// log2-sum-exp (weight 0) and D = 0.
// On operands that skiparse_rope_qk already rotated, the dq kernel copies its tiles into LDS
// with direct loads (template flag ROT) and attn_bwd_dkdv_rot_kernel replaces the dk/dv kernel:
// K' and V held in registers, the query tiles streamed into a three-deep LDS ring.
#include <mutex>
#include <type_traits>

#include "attn_common.hpp"
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

using namespace attn;

namespace {

constexpr int kDqThreads = 512;    // dq kernel: 8 wavefronts, two per SIMD
constexpr int kDqRows = 256;       // queries per dq workgroup
constexpr int kKvThreads = 512;    // dk/dv kernel: 8 wavefronts, two per SIMD
constexpr int kBwdRows = 128;      // queries (dq kernel) or keys (dk/dv kernel) per workgroup
constexpr int kBwdKN = 64;         // keys per K/V tile of the dq kernel
constexpr int kBwdQN = 64;         // queries per query tile of the dk/dv kernel

template <int D>
struct BwdLds {
    // Every tile row has this pitch: rotated Q/K rows in pair-slot order, V/dO rows in natural
    // granule order, one pad granule each.  The pad spreads 16 consecutive rows over all banks
    // (no swizzle needed), and tiles of one pitch share their operand-read addresses.
    static constexpr int kPitch = D * 2 + 16;
    // dq kernel: two K tiles and two V tiles (aliased first by the Q staging of 256 rows), the table
    static constexpr int kKTile = kBwdKN * kPitch;
    static constexpr int kVTile = kBwdKN * kPitch;
    static constexpr int kDqTiles = 2 * kKTile + 2 * kVTile;
    static constexpr int kDqTab = kDqTiles > kDqRows * kPitch ? kDqTiles : kDqRows * kPitch;
    static constexpr int kQTile = kBwdQN * kPitch;
    static constexpr int kOTile = kBwdQN * kPitch;
    // dk/dv kernel (query tiles of kQTile, kOTile): resident K' and V rows of the workgroup's keys, one Q' and one dO tile, the
    // log2-sum-exp and D of the tile, the table (the reduction at the end reuses the tiles)
    static constexpr int kKvK = 0;
    static constexpr int kKvV = kKvK + kBwdRows * kPitch;
    static constexpr int kKvQ = kKvV + kBwdRows * kPitch;
    static constexpr int kKvO = kKvQ + kQTile;
    static constexpr int kKvLd = kKvO + kOTile;
    static constexpr int kKvTab = kKvLd + 2 * kBwdQN * 4;
    static constexpr int kDkvTab = kKvTab;
    static_assert(4 * 16 * (D / 32) * 64 * 4 <= kKvLd, "the dV / dK exchange fits the tiles");
};

// 4 bytes per lane from a buffer straight into LDS: lane l's dword lands at dst + 4 l (dst
// wave-uniform; out-of-range offsets write zeros), the 4-byte form of buffer_load_to_lds16.
__device__ __forceinline__ void buffer_load_to_lds4(__amdgpu_buffer_rsrc_t r, char* dst, int off) {
    const unsigned lds_addr = (unsigned)(size_t)((__attribute__((address_space(3))) char*)dst);
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr) : "memory");
}

// 8 consecutive elements of E as a bf16x8 operand, and as floats (bf16 is exact both ways).
template <typename E>
__device__ __forceinline__ bf16x8 load8(__amdgpu_buffer_rsrc_t r, int off, float (&x)[8]) {
    ChunkRaw<E, 8> raw;
    buffer_load_dwords(r, off, raw.w);
    raw_to_f32(raw, x);
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    return v;
}

// Per-lane addresses of the LDS transpose reads that form an A operand from a tile whose rows
// are the contraction index: within each group of 16 lanes, lane i = 4t + q points at 4
// consecutive columns of row t; the instruction hands lane j the value at column c0 + j of
// each of those 4 rows.  Lanes 0-31 take rows {0-3, 8-11} and lanes 32-63 rows {4-7, 12-15}
// of every 16-row step (the order in which a 32x32 accumulator holds its rows for the B
// operand of the next product), columns 32 db + lane % 32.  Row 8 h8 + tr_row, granule
// 4 db + tr_gran, byte tr_byte; the tiles these reads serve hold their rows at BwdLds::kPitch
// in natural granule order, each row at the LDS slot tile_slot gives it.
// LDS slot of row r of a tile that is read both by 16-byte operand reads (one granule of 16
// consecutive rows per 16 lanes) and by transpose reads (4 consecutive rows x 4 granules per 32
// lanes), at the padded pitch BwdLds::kPitch (one pad granule per row): inside each block of 16
// rows, row 4 a + b (a, b < 4) sits at slot 4 b + a.  With the rows in natural order the pad
// put row r granule g on the banks of row r + 1 granule g - 1, so every transpose read took
// 4 passes (head_dim 128; 2 at 64); with this order both kinds of read touch 64 distinct banks.
// The map is its own inverse, keeps blocks of 16 in place and moves rows 0-7 of a block by 8
// to slots 2 further on, so operand addresses keep constant offsets.
__device__ __forceinline__ int tile_slot(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

struct TrLane {
    int row, gran, byte;
    __device__ __forceinline__ TrLane(int lane) {
        const int i = lane & 15;
        row = (i >> 2) + 4 * (lane >> 5);
        gran = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
        byte = (i & 1) * 8;
    }
};

// A operand (8 bf16) of one 16-row step from two transpose reads at row offsets 0 and 8.
__device__ __forceinline__ bf16x8 tr_operand(const char* p0, const char* p8) {
    const i16x4 lo = ds_read_tr16(p0);
    const i16x4 hi = ds_read_tr16(p8);
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Epilogue shared by dQ and dK: acc[db] holds the transposed gradient of one token per lane
// (column lane % 32) with rows d-slot = 32 db + 8 g + 4 (lane / 32) + jj in the pair-slot order
// of the Q/K tiles (slot 2 cp: chunk c1 of pair cp, slot 2 cp + 1: its partner c2).  Turns
// every rotate-half pair back by -theta at the token's grid position, multiplies by `scale`,
// and stores the row of token n (offsets past the slice are dropped) in natural head_dim order.
template <int D, typename E>
__device__ __forceinline__ void store_unrotated(const f32x16 (&acc)[D / 32], float scale, __amdgpu_buffer_rsrc_t out,
                                                int n, int row_bytes, const Pos& q, const char* tab, int T, int H,
                                                int phi_mul, int lane) {
    constexpr int CH = D / 16;
    constexpr int ES = E::kBytes;
    constexpr int DB = D / 32;
    const int hf = lane >> 5;
    auto entry = [&](int cp, int e) __attribute__((always_inline)) {
        const RopePair rp = rope_pair(cp);
        const int pos = rp.axis == 0 ? min(q.t, T - 1) : (rp.axis == 1 ? q.h : q.w);
        return *reinterpret_cast<const float2*>(tab + rope_tab_offset<D>(T, H, rp.axis, pos, rp.jchunk * CH + e,
                                                                        rp.axis == 2 ? phi_mul : 0));
    };
    auto store4 = [&](int chunk, int e0, const float (&y)[4]) __attribute__((always_inline)) {
        const int off = n * row_bytes + (chunk * CH + e0) * ES;
        if constexpr (ES == 2) {
            const u32x2 v2 = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
            __builtin_amdgcn_raw_buffer_store_b64(v2, out, off, 0, 0);
        } else {
            const u32x4 v4 = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
            __builtin_amdgcn_raw_buffer_store_b128(v4, out, off, 0, 0);
        }
    };
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        if constexpr (CH == 8) {
            // granule 4 db + g is slot 4 db + g: g even holds c1 elements, g + 1 their partners
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
                const int cp = 2 * db + g / 2;
                const RopePair rp = rope_pair(cp);
                float y1[4], y2[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int e = 4 * hf + jj;
                    const float2 cs = entry(cp, e);
                    const float a1 = acc[db][4 * g + jj], a2 = acc[db][4 * (g + 1) + jj];
                    y1[jj] = (a1 * cs.x + a2 * cs.y) * scale;
                    y2[jj] = (a2 * cs.x - a1 * cs.y) * scale;
                }
                store4(rp.c1, 4 * hf, y1);
                store4(rp.c2, 4 * hf, y2);
            }
        } else {
            // CH = 4: slot 8 db + 2 g + hf, so a c1 element's partner sits in the lane 32 away
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cp = 4 * db + g;
                const RopePair rp = rope_pair(cp);
                float y[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float own = acc[db][4 * g + jj];
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(own), __float_as_uint(own), false, false);
                    const float other = __uint_as_float(hf ? sw[0] : sw[1]);
                    const float a1 = hf ? other : own, a2 = hf ? own : other;
                    const float2 cs = entry(cp, jj);
                    y[jj] = (hf ? (a2 * cs.x - a1 * cs.y) : (a1 * cs.x + a2 * cs.y)) * scale;
                }
                store4(hf ? rp.c2 : rp.c1, 0, y);
            }
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------------------------
// KDIV: sparse_k divides the tile height, so row r + tile of a scope is token n(r) + tile * k
// in both modes and the load cursors and grid positions advance by constants.
//
// 8 wavefronts (two per SIMD) of 32 queries.  Each 64-key tile is processed one 32-key block
// at a time (S^T and dP^T of the block, its dZ^T, its two 16-key steps of dQ'^T), so only one
// block's score accumulators are live and a wavefront fits in 256 VGPRs: the MFMAs take their
// accumulators in VGPRs (no AGPR copies) and the two wavefronts of a SIMD hide each other's
// LDS and dependency latency.
// One (row, RoPE chunk pair) staging task for operands that are already rotated (and, for q,
// scaled): the output of skiparse_rope_qk.  The pair's two chunks are moved unchanged into the
// pair-slot order, so the LDS rows hold exactly what stage_rotated_pair computes from q, k.
template <int D>
__device__ __forceinline__ void stage_copied_pair(__amdgpu_buffer_rsrc_t r, int off, const RopePair& rp, int cp,
                                                  char* lds_row) {
    constexpr int CH = D / 16;
    static_assert(CH == 8, "rotated operands: head_dim 128");
    uint32_t w1[4], w2[4];
    buffer_load_dwords(r, off + rp.c1 * CH * 2, w1);
    buffer_load_dwords(r, off + rp.c2 * CH * 2, w2);
    *reinterpret_cast<u32x4*>(lds_row + 2 * cp * CH * 2) = u32x4{w1[0], w1[1], w1[2], w1[3]};
    *reinterpret_cast<u32x4*>(lds_row + (2 * cp + 1) * CH * 2) = u32x4{w2[0], w2[1], w2[2], w2[3]};
}

template <int D, typename E, bool KDIV, bool ROT>
__global__ void __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(AttnBwdParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef BwdLds<D> L;
    constexpr int CH = D / 16;
    constexpr int KS = D / 16;        // 16-deep k-steps over head_dim
    constexpr int DB = D / 32;        // 32-row blocks of head_dim
    constexpr int KB = kBwdKN / 32;   // 32-key blocks per tile
    constexpr int ES = E::kBytes;
    constexpr int G = D / 8;          // 16-byte granules per V row (bf16)
    constexpr int kVPer = kBwdKN * G / kDqThreads;    // V granules per thread per tile
    static_assert(kBwdKN * 8 == kDqThreads, "one K staging task per thread per tile");
    char* ktile = lds;
    char* vtile = lds + 2 * L::kKTile;
    char* tab = lds + L::kDqTab;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = work % a.dq_tiles;
    const int sc = work / a.dq_tiles;
    const int s = sc % a.sparse_k;
    const int bh = sc / a.sparse_k;
    const int head = bh % a.heads;
    const int b = bh / a.heads;
    const int64_t k_ = a.sparse_k;
    const int row_bytes = a.heads * D * ES;
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * ES;
    const int slice_bytes = a.N * row_bytes - head * D * ES;
    auto rsrc = [&](const void* base) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const char*>(base) + slice), (short)0,
                                                 slice_bytes, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t qbuf = rsrc(a.q), kbuf = rsrc(a.k), vbuf = rsrc(a.v), obuf = rsrc(a.o),
                                 dobuf = rsrc(a.dout), dqbuf = rsrc(a.dq);
    const int64_t vec0 = ((int64_t)b * a.heads + head) * a.N;   // (b, head) row of lse / delta
    const int HW = a.H * a.W;
    auto pos_of = [&](int nn) __attribute__((always_inline)) {
        Pos q;
        q.t = nn / HW; q.h = (nn / a.W) % a.H; q.w = nn % a.W;
        return q;
    };

    build_banked_rope_table<D>(tab, a.T, a.H, a.W, a.phi_mul);
    const int cp = tid & 7;
    const RopePair rp = rope_pair(cp);
    __syncthreads();

    // ---- Q tile: rotated, scaled by log2(e)/sqrt(d), through LDS into B-operand registers ----
#pragma unroll 2
    for (int it = 0; it < kDqRows * 8 / kDqThreads; ++it) {
        const int r = (tid >> 3) + it * (kDqThreads / 8);
        const int n = (int)scope_token(qt * kDqRows + r, s, k_, a.mode);   // >= N past the scope end
        if constexpr (ROT)
            stage_copied_pair<D>(qbuf, n * row_bytes, rp, cp, ktile + r * L::kPitch);
        else
            stage_rotated_pair<D, E>(qbuf, n * row_bytes, rp, cp, tab, a.T, a.H, pos_of(n), a.phi_mul, a.scale_log2,
                                     ktile + r * L::kPitch);
    }
    __syncthreads();
    bf16x8 qreg[KS];
    {
        const char* qrow = ktile + (wave * 32 + l32) * L::kPitch;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + hf) * 16);
    }
    __syncthreads();   // the staging rows become K tiles

    // ---- this lane's query: dO as the B operand of dP^T = V dO^T (natural order), D, LSE ----
    const int pq = qt * kDqRows + wave * 32 + l32;
    const int nq = (int)scope_token(pq, s, k_, a.mode);
    const bool qvalid = pq < a.L;
    bf16x8 doreg[KS];
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int off = nq * row_bytes + (2 * ks + hf) * 8 * ES;
        float xd[8], xo[8];
        doreg[ks] = load8<E>(dobuf, off, xd);
        load8<E>(obuf, off, xo);
#pragma unroll
        for (int e = 0; e < 8; ++e) dsum += xd[e] * xo[e];
    }
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
        dsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float dq_d = qvalid ? dsum : 0.f;
    if (qvalid && hf == 0) a.delta[vec0 + nq] = dq_d;
    const float lse_q = qvalid ? a.lse[vec0 + nq] : 0.f;

    // ---- K/V tiles: loaded into registers one tile ahead, staged at the end of a tile ----
    const int krow = tid >> 3;   // K staging task: row krow, chunk pair cp
    ChunkRaw<E, CH> kraw[2];
    Pos kpos;
    uint32_t vraw[kVPer][4];
    // cursors: token rows of this thread's K and V rows in the tile being loaded (KDIV: advanced
    // by a constant per tile, grid positions with carries)
    int kn, vn[kVPer];
    const int tile_dn = kBwdKN * a.sparse_k;
    const int dt = tile_dn / HW, drem = tile_dn % HW;
    const int dh = drem / a.W, dw = drem % a.W;
    auto set_rows = [&](int t) __attribute__((always_inline)) {
        kn = (int)scope_token(t * kBwdKN + krow, s, k_, a.mode);
        kpos = pos_of(kn);
#pragma unroll
        for (int i = 0; i < kVPer; ++i) vn[i] = (int)scope_token(t * kBwdKN + (tid + kDqThreads * i) / G, s, k_, a.mode);
    };
    auto advance_rows = [&](int t) __attribute__((always_inline)) {   // to tile t, from t - 1
        if constexpr (KDIV) {
            kn += tile_dn;
            int w = kpos.w + dw, c = w >= a.W;
            kpos.w = w - (c ? a.W : 0);
            int h = kpos.h + dh + c;
            c = h >= a.H;
            kpos.h = h - (c ? a.H : 0);
            kpos.t += dt + c;
#pragma unroll
            for (int i = 0; i < kVPer; ++i) vn[i] += tile_dn;
        } else {
            set_rows(t);
        }
    };
    auto load_kv = [&]() __attribute__((always_inline)) {
        buffer_load_dwords(kbuf, kn * row_bytes + rp.c1 * CH * ES, kraw[0].w);
        buffer_load_dwords(kbuf, kn * row_bytes + rp.c2 * CH * ES, kraw[1].w);
#pragma unroll
        for (int i = 0; i < kVPer; ++i)
            buffer_load_8_as_bf16x2<E>(vbuf, vn[i] * row_bytes + ((tid + kDqThreads * i) % G) * 8 * ES, vraw[i]);
    };
    auto store_kv = [&](int buf) __attribute__((always_inline)) {
        char* kd = ktile + buf * L::kKTile;
        char* dst = kd + tile_slot(krow) * L::kPitch;
        if constexpr (ROT) {
            // already rotated: the chunks move unchanged
            *reinterpret_cast<u32x4*>(dst + 2 * cp * CH * 2) = u32x4{kraw[0].w[0], kraw[0].w[1], kraw[0].w[2], kraw[0].w[3]};
            *reinterpret_cast<u32x4*>(dst + (2 * cp + 1) * CH * 2) = u32x4{kraw[1].w[0], kraw[1].w[1], kraw[1].w[2], kraw[1].w[3]};
        } else {
            float x1[CH], x2[CH];
            raw_to_f32(kraw[0], x1);
            raw_to_f32(kraw[1], x2);
            const int pos = rp.axis == 0 ? min(kpos.t, a.T - 1) : (rp.axis == 1 ? kpos.h : kpos.w);
            const char* row = tab + rope_tab_offset<D>(a.T, a.H, rp.axis, pos, rp.jchunk * CH, rp.axis == 2 ? a.phi_mul : 0);
            f32x4 cs[CH / 2];
#pragma unroll
            for (int j = 0; j < CH / 2; ++j) cs[j] = *reinterpret_cast<const f32x4*>(row + 16 * j);
            rope_rotate_cs<CH>(x1, x2, cs);
            store_rotated_chunks<CH>(dst + 2 * cp * CH * 2, dst + (2 * cp + 1) * CH * 2, x1, x2);
        }
        char* vd = vtile + buf * L::kVTile;
#pragma unroll
        for (int i = 0; i < kVPer; ++i) {
            const int idx = tid + kDqThreads * i;
            const int r = idx / G;
            *reinterpret_cast<u32x4*>(vd + tile_slot(r) * L::kPitch + (idx % G) * 16) =
                u32x4{vraw[i][0], vraw[i][1], vraw[i][2], vraw[i][3]};
        }
    };

    // Rotated operands (ROT): the K and V tiles need no arithmetic, so they are copied into LDS
    // by loads that write LDS directly.  The padded K tile is 17 pieces of 1 KiB: in piece p,
    // lane l fills granule 64 p + l, i.e. slot (64 p + l) mod 17 of row (64 p + l) div 17, with
    // the chunk that the pair-slot order puts there (slot 16, the pad, takes chunk 0 and is
    // never read).  Wave w moves pieces w and w + 8, wave 0 also piece 16.  The V tile has the
    // same pitch and pieces with each slot's own chunk; wave 1 moves its piece 16.
    static_assert(!ROT || (kBwdKN * L::kPitch == 17 * 1024 && L::kVTile == 17 * 1024 && kDqThreads == 512),
                  "tile pieces of the direct loads");
    int kdo[3], vdo[3];
    auto set_dma_rows = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int gi = 64 * (j < 2 ? wave + 8 * j : 16) + lane;
            const int row = tile_slot(gi / 17), slot = gi % 17;   // the tile row that LDS row gi / 17 holds
            const RopePair sp = rope_pair((slot >> 1) & 7);
            const int c = slot == 16 ? 0 : ((slot & 1) ? sp.c2 : sp.c1);
            kdo[j] = (int)scope_token(t * kBwdKN + row, s, k_, a.mode) * row_bytes + c * 16;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int gi = 64 * (j < 2 ? wave + 8 * j : 16) + lane;
            const int row = tile_slot(gi / 17), slot = gi % 17;
            vdo[j] = (int)scope_token(t * kBwdKN + row, s, k_, a.mode) * row_bytes + (slot == 16 ? 0 : slot) * 16;
        }
    };
    auto advance_dma_rows = [&](int t) __attribute__((always_inline)) {   // to tile t, from t - 1
        if constexpr (KDIV) {
#pragma unroll
            for (int j = 0; j < 3; ++j) kdo[j] += tile_dn * row_bytes;
#pragma unroll
            for (int j = 0; j < 3; ++j) vdo[j] += tile_dn * row_bytes;
        } else {
            set_dma_rows(t);
        }
    };
    auto dma_kv = [&](int buf) __attribute__((always_inline)) {
        char* kd = ktile + buf * L::kKTile;
        char* vd = vtile + buf * L::kVTile;
        buffer_load_to_lds16(kbuf, kd + wave * 1024, kdo[0]);
        buffer_load_to_lds16(kbuf, kd + (wave + 8) * 1024, kdo[1]);
        if (wave == 0) buffer_load_to_lds16(kbuf, kd + 16 * 1024, kdo[2]);
        buffer_load_to_lds16(vbuf, vd + wave * 1024, vdo[0]);
        buffer_load_to_lds16(vbuf, vd + (wave + 8) * 1024, vdo[1]);
        if (wave == 1) buffer_load_to_lds16(vbuf, vd + 16 * 1024, vdo[2]);
    };

    const TrLane tr(lane);
    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) dqacc[db][x] = 0.f;
    const int nt = (a.L + kBwdKN - 1) / kBwdKN;
    set_rows(0);
    if constexpr (ROT) {
        set_dma_rows(0);
        dma_kv(0);
        wait_vm_loads();
    } else {
        load_kv();
        store_kv(0);
    }
    __syncthreads();
    constexpr int kR = 4;   // depth of the operand rings
    // one key tile; `masked`: the last tile, whose keys past the end of the scope start at -inf
    // (a separate instantiation, peeled out of the loop, so the other tiles carry no masking)
    auto tile = [&](int t, auto masked) __attribute__((always_inline)) {
        if (t + 1 < nt) {
            if constexpr (ROT) {
                // buffer (t + 1) & 1 held tile t - 1, whose readers all passed the last barrier
                advance_dma_rows(t + 1);
                dma_kv((t + 1) & 1);
            } else {
                advance_rows(t + 1);
                load_kv();
            }
        }
        const char* kc = ktile + (t & 1) * L::kKTile;
        const char* vc = vtile + (t & 1) * L::kVTile;
        const int valid = a.L - t * kBwdKN;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            // S^T = K Q'^T and dP^T = V dO^T of the 32-key block, operands through rings
            f32x16 sacc, dpacc;
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                if constexpr (decltype(masked)::value)
                    sacc[x] = kb * 32 + 8 * (x >> 2) + 4 * hf + (x & 3) < valid ? -lse_q : -__builtin_inff();
                else
                    sacc[x] = -lse_q;
                dpacc[x] = 0.f;
            }
            {
                const int r = tile_slot(kb * 32 + l32);
                auto kop = [&](int ks) __attribute__((always_inline)) {
                    return *reinterpret_cast<const bf16x8*>(kc + r * L::kPitch + (2 * ks + hf) * 16);
                };
                auto vop = [&](int ks) __attribute__((always_inline)) {
                    return *reinterpret_cast<const bf16x8*>(vc + r * L::kPitch + (2 * ks + hf) * 16);
                };
                bf16x8 ka[kR], va[kR];
#pragma unroll
                for (int ks = 0; ks < kR - 1; ++ks) {
                    ka[ks] = kop(ks);
                    va[ks] = vop(ks);
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + kR - 1 < KS) {
                        ka[(ks + kR - 1) % kR] = kop(ks + kR - 1);
                        va[(ks + kR - 1) % kR] = vop(ks + kR - 1);
                    }
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks % kR], qreg[ks], sacc, 0, 0, 0);
                    dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks % kR], doreg[ks], dpacc, 0, 0, 0);
                }
            }
            // dZ^T = P^T * (dP^T - D) of the block as two bf16 B operands (keys 8 g + 4 hf + jj
            // sit in 16-key step g / 2, slot 4 (g % 2) + jj)
            bf16x8 dzb[2];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int x = 4 * g + jj;
                    const float p = __builtin_amdgcn_exp2f(sacc[x]);
                    dzb[g >> 1][(g & 1) * 4 + jj] = (__bf16)(p * (dpacc[x] - dq_d));
                }
            // dQ'^T += K^T dZ^T over the block's two 16-key steps, K^T from transpose reads
            {
                constexpr int NST = 2 * DB;
                auto top = [&](int st) __attribute__((always_inline)) {
                    const char* base = kc + tile_slot(32 * kb + 16 * (st / DB) + tr.row) * L::kPitch + (4 * (st % DB) + tr.gran) * 16 + tr.byte;
                    return tr_operand(base, base + 2 * L::kPitch);   // rows 8 further on: slots 2 further on
                };
                bf16x8 ta[kR];
#pragma unroll
                for (int st = 0; st < kR - 1; ++st) ta[st] = top(st);
#pragma unroll
                for (int st = 0; st < NST; ++st) {
                    if (st + kR - 1 < NST) ta[(st + kR - 1) % kR] = top(st + kR - 1);
                    dqacc[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[st % kR], dzb[st / DB], dqacc[st % DB], 0, 0, 0);
                }
            }
        }
        if constexpr (!ROT) {
            if (t + 1 < nt) store_kv((t + 1) & 1);
        }
        wait_vm_loads();
        __syncthreads();
    };
    for (int t = 0; t < nt - 1; ++t) tile(t, std::false_type{});
    tile(nt - 1, std::true_type{});

    // ---- epilogue: dq = c * (transposed RoPE of dQ'), to the query's token ----
    if (!qvalid) return;
    store_unrotated<D, E>(dqacc, a.scale, dqbuf, nq, row_bytes, pos_of(nq), tab, a.T, a.H, a.phi_mul, lane);
}

// ---------------------------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------------------------
// KDIV: sparse_k divides the query-tile height (cursors advance by constants, as in the dq kernel)
//
// 8 wavefronts (two per SIMD).  Wavefronts w and w + 4 (one SIMD) own the same 32 keys and take
// the two 32-query halves of every 64-query tile; at the end they add their partial dV and dK
// through LDS.  Every MFMA operand comes from LDS (the K', V rows of the workgroup's 128 keys
// stay resident; the Q', dO tile is staged once per query tile), so a wavefront fits in 256
// VGPRs and its accumulators stay in VGPRs.
template <int D, typename E, bool KDIV>
__global__ void __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_kernel(AttnBwdParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef BwdLds<D> L;
    constexpr int CH = D / 16;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int ES = E::kBytes;
    constexpr int G = D / 8;                           // 16-byte granules per dO / V row (bf16)
    constexpr int kOPer = kBwdQN * G / kKvThreads;     // dO granules per thread per tile
    constexpr int kQPer = kBwdQN * 8 / kKvThreads;     // Q staging tasks per thread per tile
    constexpr int kKPer = kBwdRows * 8 / kKvThreads;   // K staging tasks per thread
    constexpr int kVPer = kBwdRows * G / kKvThreads;   // V granules per thread
    char* kres = lds + L::kKvK;       // resident K' rows of the workgroup's keys
    char* vres = lds + L::kKvV;       // resident V rows
    char* qtile = lds + L::kKvQ;      // Q' rows of the current query tile
    char* otile = lds + L::kKvO;      // dO rows of the current query tile
    float* ldt = reinterpret_cast<float*>(lds + L::kKvLd);   // [0, QN): LSE, [QN, 2 QN): D
    char* tab = lds + L::kKvTab;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kgrp = wave & 3, qhalf = wave >> 2;
    const int l32 = lane & 31, hf = lane >> 5;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = work % a.tiles;
    const int sc = work / a.tiles;
    const int s = sc % a.sparse_k;
    const int bh = sc / a.sparse_k;
    const int head = bh % a.heads;
    const int b = bh / a.heads;
    const int64_t k_ = a.sparse_k;
    const int row_bytes = a.heads * D * ES;
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * ES;
    const int slice_bytes = a.N * row_bytes - head * D * ES;
    auto rsrc = [&](const void* base) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const char*>(base) + slice), (short)0,
                                                 slice_bytes, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t qbuf = rsrc(a.q), kbuf = rsrc(a.k), vbuf = rsrc(a.v), dobuf = rsrc(a.dout),
                                 dkbuf = rsrc(a.dk), dvbuf = rsrc(a.dv);
    const int64_t vec0 = ((int64_t)b * a.heads + head) * a.N;
    const int HW = a.H * a.W;
    auto pos_of = [&](int nn) __attribute__((always_inline)) {
        Pos q;
        q.t = nn / HW; q.h = (nn / a.W) % a.H; q.w = nn % a.W;
        return q;
    };

    build_banked_rope_table<D>(tab, a.T, a.H, a.W, a.phi_mul);
    const int cp = tid & 7;
    const RopePair rp = rope_pair(cp);
    __syncthreads();

    // ---- resident K' (rotated, unscaled) and V rows of the workgroup's 128 keys ----
#pragma unroll
    for (int it = 0; it < kKPer; ++it) {
        const int r = (tid >> 3) + it * (kKvThreads / 8);
        const int n = (int)scope_token(kt * kBwdRows + r, s, k_, a.mode);
        stage_rotated_pair<D, E>(kbuf, n * row_bytes, rp, cp, tab, a.T, a.H, pos_of(n), a.phi_mul, 1.0f,
                                 kres + r * L::kPitch);
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
        const int idx = tid + kKvThreads * i;
        const int r = idx / G;
        const int n = (int)scope_token(kt * kBwdRows + r, s, k_, a.mode);
        uint32_t w[4];
        buffer_load_8_as_bf16x2<E>(vbuf, n * row_bytes + (idx % G) * 8 * ES, w);
        *reinterpret_cast<u32x4*>(vres + r * L::kPitch + (idx % G) * 16) = u32x4{w[0], w[1], w[2], w[3]};
    }
    const int pk = kt * kBwdRows + kgrp * 32 + l32;   // this lane's key (the B-operand column)
    const int nk = (int)scope_token(pk, s, k_, a.mode);
    const int kr = kgrp * 32 + l32;                    // its row in the resident tiles

    // ---- query tiles: loaded into registers one tile ahead, staged at the start of a tile ----
    const int qrow = tid >> 3;   // Q staging task: row qrow, chunk pair cp
    static_assert(kQPer == 1, "one Q staging task per thread per tile");
    ChunkRaw<E, CH> qraw[2];
    Pos qpos;
    uint32_t oraw[kOPer][4];
    float ldv = 0.f;
    int qn, on[kOPer], ln;
    const int tile_dn = kBwdQN * a.sparse_k;
    const int dt = tile_dn / HW, drem = tile_dn % HW;
    const int dh = drem / a.W, dw = drem % a.W;
    auto set_rows = [&](int i) __attribute__((always_inline)) {
        qn = (int)scope_token(i * kBwdQN + qrow, s, k_, a.mode);
        qpos = pos_of(qn);
#pragma unroll
        for (int j = 0; j < kOPer; ++j) on[j] = (int)scope_token(i * kBwdQN + (tid + kKvThreads * j) / G, s, k_, a.mode);
        ln = (int)scope_token(i * kBwdQN + (tid % kBwdQN), s, k_, a.mode);
    };
    auto advance_rows = [&](int i) __attribute__((always_inline)) {   // to tile i, from i - 1
        if constexpr (KDIV) {
            qn += tile_dn;
            int w = qpos.w + dw, c = w >= a.W;
            qpos.w = w - (c ? a.W : 0);
            int h = qpos.h + dh + c;
            c = h >= a.H;
            qpos.h = h - (c ? a.H : 0);
            qpos.t += dt + c;
#pragma unroll
            for (int j = 0; j < kOPer; ++j) on[j] += tile_dn;
            ln += tile_dn;
        } else {
            set_rows(i);
        }
    };
    auto load_q = [&](int i) __attribute__((always_inline)) {
        buffer_load_dwords(qbuf, qn * row_bytes + rp.c1 * CH * ES, qraw[0].w);
        buffer_load_dwords(qbuf, qn * row_bytes + rp.c2 * CH * ES, qraw[1].w);
#pragma unroll
        for (int j = 0; j < kOPer; ++j)
            buffer_load_8_as_bf16x2<E>(dobuf, on[j] * row_bytes + ((tid + kKvThreads * j) % G) * 8 * ES, oraw[j]);
        if (tid < 2 * kBwdQN) {
            const int p = i * kBwdQN + (tid % kBwdQN);
            ldv = tid < kBwdQN ? (p < a.L ? a.lse[vec0 + ln] : __builtin_inff())
                               : (p < a.L ? a.delta[vec0 + ln] : 0.f);
        }
    };
    auto store_q = [&]() __attribute__((always_inline)) {
        char* dst = qtile + tile_slot(qrow) * L::kPitch;
        {
            float x1[CH], x2[CH];
            raw_to_f32(qraw[0], x1);
            raw_to_f32(qraw[1], x2);
            const int pos = rp.axis == 0 ? min(qpos.t, a.T - 1) : (rp.axis == 1 ? qpos.h : qpos.w);
            const char* row = tab + rope_tab_offset<D>(a.T, a.H, rp.axis, pos, rp.jchunk * CH, rp.axis == 2 ? a.phi_mul : 0);
            f32x4 cs[CH / 2];
#pragma unroll
            for (int j = 0; j < CH / 2; ++j) cs[j] = *reinterpret_cast<const f32x4*>(row + 16 * j);
            rope_rotate_cs<CH>(x1, x2, cs);
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                x1[e] *= a.scale_log2;
                x2[e] *= a.scale_log2;
            }
            store_rotated_chunks<CH>(dst + 2 * cp * CH * 2, dst + (2 * cp + 1) * CH * 2, x1, x2);
        }
#pragma unroll
        for (int j = 0; j < kOPer; ++j) {
            const int idx = tid + kKvThreads * j;
            const int r = idx / G;
            *reinterpret_cast<u32x4*>(otile + tile_slot(r) * L::kPitch + (idx % G) * 16) =
                u32x4{oraw[j][0], oraw[j][1], oraw[j][2], oraw[j][3]};
        }
        if (tid < 2 * kBwdQN) ldt[tid] = ldv;
    };

    const TrLane tr(lane);
    f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            dvacc[db][x] = 0.f;
            dkacc[db][x] = 0.f;
        }
    constexpr int kR = 3;   // depth of the operand rings
    const int qb0 = 32 * qhalf;   // this wavefront's query rows in each tile
    const int nq = (a.L + kBwdQN - 1) / kBwdQN;
    set_rows(0);
    load_q(0);
    for (int i = 0; i < nq; ++i) {
        wait_vm_loads();
        __syncthreads();           // every read of the previous tile's Q', dO is done
        store_q();
        __syncthreads();
        if (i + 1 < nq) {
            advance_rows(i + 1);
            load_q(i + 1);
        }
        // start values -LSE and D of the queries qb0 + 8 g + 4 hf + jj this lane's accumulator rows hold
        f32x16 sacc, dpacc;
        float dd[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(ldt + qb0 + 8 * g + 4 * hf);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(ldt + kBwdQN + qb0 + 8 * g + 4 * hf);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                sacc[4 * g + jj] = -l4[jj];
                dd[4 * g + jj] = d4[jj];
                dpacc[4 * g + jj] = 0.f;
            }
        }
        // S = Q' K'^T and dP = dO V^T of the 32-query block, all four operands from LDS
        {
            const int r = tile_slot(qb0 + l32);
            auto qop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(qtile + r * L::kPitch + (2 * ks + hf) * 16);
            };
            auto oop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(otile + r * L::kPitch + (2 * ks + hf) * 16);
            };
            auto kop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(kres + kr * L::kPitch + (2 * ks + hf) * 16);
            };
            auto vop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(vres + kr * L::kPitch + (2 * ks + hf) * 16);
            };
            bf16x8 qa[kR], oa[kR], kb_[kR], vb_[kR];
#pragma unroll
            for (int ks = 0; ks < kR - 1; ++ks) {
                qa[ks] = qop(ks); oa[ks] = oop(ks); kb_[ks] = kop(ks); vb_[ks] = vop(ks);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + kR - 1 < KS) {
                    const int n1 = (ks + kR - 1) % kR;
                    qa[n1] = qop(ks + kR - 1); oa[n1] = oop(ks + kR - 1);
                    kb_[n1] = kop(ks + kR - 1); vb_[n1] = vop(ks + kR - 1);
                }
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks % kR], kb_[ks % kR], sacc, 0, 0, 0);
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[ks % kR], vb_[ks % kR], dpacc, 0, 0, 0);
            }
        }
        // P and dZ as bf16 B operands (query qb0 + 8 g + 4 hf + jj in 16-query step g / 2, slot
        // 4 (g % 2) + jj)
        bf16x8 pbb[2], dzb[2];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int x = 4 * g + jj;
                const float p = __builtin_amdgcn_exp2f(sacc[x]);
                pbb[g >> 1][(g & 1) * 4 + jj] = (__bf16)p;
                dzb[g >> 1][(g & 1) * 4 + jj] = (__bf16)(p * (dpacc[x] - dd[x]));
            }
        // dV^T += dO^T P and dK^T += Q'^T dZ over the block's two 16-query steps
        {
            constexpr int NST = 2 * DB;
            auto dop = [&](int st) __attribute__((always_inline)) {
                const int kk = st / DB, db = st % DB;
                const char* ob = otile + tile_slot(qb0 + 16 * kk + tr.row) * L::kPitch + (4 * db + tr.gran) * 16 + tr.byte;
                return tr_operand(ob, ob + 2 * L::kPitch);
            };
            auto qtop = [&](int st) __attribute__((always_inline)) {
                const int kk = st / DB, db = st % DB;
                const char* qb = qtile + tile_slot(qb0 + 16 * kk + tr.row) * L::kPitch + (4 * db + tr.gran) * 16 + tr.byte;
                return tr_operand(qb, qb + 2 * L::kPitch);
            };
            bf16x8 da[kR], ka2[kR];
#pragma unroll
            for (int st = 0; st < kR - 1; ++st) {
                da[st] = dop(st);
                ka2[st] = qtop(st);
            }
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                if (st + kR - 1 < NST) {
                    da[(st + kR - 1) % kR] = dop(st + kR - 1);
                    ka2[(st + kR - 1) % kR] = qtop(st + kR - 1);
                }
                dvacc[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[st % kR], pbb[st / DB], dvacc[st % DB], 0, 0, 0);
                dkacc[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka2[st % kR], dzb[st / DB], dkacc[st % DB], 0, 0, 0);
            }
        }
    }

    // ---- the two query halves' partial sums meet in LDS (the tiles are free now) ----
    float* red = reinterpret_cast<float*>(lds);   // [kgrp][16 * DB values][64 lanes]
    auto exchange = [&](f32x16 (&acc)[DB]) __attribute__((always_inline)) {
        __syncthreads();
        if (qhalf == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) red[(kgrp * 16 * DB + db * 16 + x) * 64 + lane] = acc[db][x];
        }
        __syncthreads();
        if (qhalf == 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) acc[db][x] += red[(kgrp * 16 * DB + db * 16 + x) * 64 + lane];
        }
    };
    exchange(dvacc);
    exchange(dkacc);

    // ---- epilogue (query half 0): dv rows, and dk = (transposed RoPE of dK') / log2(e) ----
    if (qhalf != 0 || pk >= a.L) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + 8 * g + 4 * hf;
            const float y0 = dvacc[db][4 * g], y1 = dvacc[db][4 * g + 1];
            const float y2 = dvacc[db][4 * g + 2], y3 = dvacc[db][4 * g + 3];
            if constexpr (ES == 2) {
                const u32x2 v2 = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                __builtin_amdgcn_raw_buffer_store_b64(v2, dvbuf, nk * row_bytes + d0 * 2, 0, 0);
            } else {
                const u32x4 v4 = {__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3)};
                __builtin_amdgcn_raw_buffer_store_b128(v4, dvbuf, nk * row_bytes + d0 * 4, 0, 0);
            }
        }
    store_unrotated<D, E>(dkacc, 0.69314718055994530942f, dkbuf, nk, row_bytes, pos_of(nk), tab, a.T, a.H, a.phi_mul, lane);
}

// ---------------------------------------------------------------------------------------------
// dK and dV on rotated operands (head_dim 128, bf16)
// ---------------------------------------------------------------------------------------------
// The products of attn_bwd_dkdv_kernel, in the same order, for the q' (rotated, scaled) and k'
// (rotated) that skiparse_rope_qk writes.  With nothing to convert or rotate on the way in:
// - the K' and V rows of a wavefront's 32 keys go from memory straight into registers as MFMA
//   B operands, read once instead of from LDS on every query tile;
// - the query tiles (Q' rows in pair-slot order, dO rows in natural order, both with the
//   272-byte pitch whose pad granule spreads 16 rows over all banks, log2-sum-exp, D) go from
//   memory straight into a ring of three LDS buffers, two tiles ahead of their use, with one
//   barrier per tile.  Both tiles share one row pitch and so one set of read addresses.
// Rows past the end of the scope map to tokens past the slice and read as zeros, so their
// log2-sum-exp and D are 0 (not +inf and 0): with Q' = dO = 0 their P is 1 but dP = 0 and
// dZ = 0, and every product they enter adds exactly zero.
struct RotKvLds {
    static constexpr int kQ = 17 * 1024;            // 64 Q' rows of 272 bytes: 17 pieces of 1 KiB
    static constexpr int kO = 17 * 1024;            // 64 dO rows of 272 bytes
    static constexpr int kBuf = kQ + kO + 2 * 256;  // + log2-sum-exp and D of the 64 queries
    static constexpr int kNB = 3;
    static constexpr int kTab = kNB * kBuf;         // the RoPE table (read by the epilogue only)
};

template <bool KDIV>
__global__ void __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_rot_kernel(AttnBwdParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    constexpr int D = 128;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int kPitch = D * 2 + 16;       // Q' and dO rows: 16 granules and a pad granule
    typedef RotKvLds R;
    static_assert(kBwdQN == 64 && kBwdQN * kPitch == R::kQ && R::kO == R::kQ && kKvThreads == 512,
                  "tile pieces of the direct loads");
    static_assert(4 * 16 * DB * 64 * 4 <= R::kTab, "the dV / dK exchange fits the ring");
    char* tab = lds + R::kTab;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kgrp = wave & 3, qhalf = wave >> 2;
    const int l32 = lane & 31, hf = lane >> 5;
    const int work = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = work % a.tiles;
    const int sc = work / a.tiles;
    const int s = sc % a.sparse_k;
    const int bh = sc / a.sparse_k;
    const int head = bh % a.heads;
    const int b = bh / a.heads;
    const int64_t k_ = a.sparse_k;
    const int row_bytes = a.heads * D * 2;
    const int64_t slice = ((int64_t)b * a.N * a.heads + head) * D * 2;
    const int slice_bytes = a.N * row_bytes - head * D * 2;
    auto rsrc = [&](const void* base, int64_t off, int bytes) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const char*>(base) + off), (short)0, bytes,
                                                 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t qbuf = rsrc(a.q, slice, slice_bytes), kbuf = rsrc(a.k, slice, slice_bytes),
                                 vbuf = rsrc(a.v, slice, slice_bytes), dobuf = rsrc(a.dout, slice, slice_bytes),
                                 dkbuf = rsrc(a.dk, slice, slice_bytes), dvbuf = rsrc(a.dv, slice, slice_bytes);
    const int64_t vec0 = ((int64_t)b * a.heads + head) * a.N;   // (b, head) row of lse / delta
    const __amdgpu_buffer_rsrc_t lbuf = rsrc(a.lse, vec0 * 4, a.N * 4), dlbuf = rsrc(a.delta, vec0 * 4, a.N * 4);
    const int HW = a.H * a.W;

    build_banked_rope_table<D>(tab, a.T, a.H, a.W, a.phi_mul);

    // ---- K' and V of this lane's key as B operands: k-step ks takes chunk c1 (lanes 0-31) or
    // c2 (lanes 32-63) of RoPE pair ks for K', natural granule 2 ks + hf for V ----
    const int pk = kt * kBwdRows + kgrp * 32 + l32;
    const int nk = (int)scope_token(pk, s, k_, a.mode);
    bf16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const RopePair rp = rope_pair(ks);
        uint32_t w[4];
        buffer_load_dwords(kbuf, nk * row_bytes + (hf ? rp.c2 : rp.c1) * 16, w);
        kreg[ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        buffer_load_dwords(vbuf, nk * row_bytes + (2 * ks + hf) * 16, w);
        vreg[ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
    }

    // ---- query tiles, straight into LDS buffer i mod 3 ----
    // Each tile is 17 pieces of 1 KiB: in piece p, lane l fills granule 64 p + l, i.e. slot
    // (64 p + l) mod 17 of row (64 p + l) div 17 (slot 16, the pad, takes chunk 0 and is never
    // read).  A Q' slot holds the chunk that the pair-slot order puts there, a dO slot the chunk
    // of its own number.  Wave w moves pieces w and w + 8 of both tiles; wave 0 also Q' piece 16,
    // wave 1 dO piece 16, wave 2 the tile's log2-sum-exp and wave 3 its D.
    const int tile_dn = kBwdQN * a.sparse_k;
    int qdo[2], odo[2], xdo = 0;
    // the lane index, recomputed where it is used: without KDIV the offsets are rebuilt every
    // tile, and values derived from a lane index kept since the start would hold registers the
    // loop does not have
    auto opaque_lane = [&]() __attribute__((always_inline)) {
        if constexpr (KDIV) return lane;
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        return l;
    };
    auto piece_off = [&](int i, int p, bool pair_slot) __attribute__((always_inline)) {
        const int gi = 64 * p + opaque_lane();
        const int row = tile_slot(gi / 17), slot = gi % 17;   // the tile row that LDS row gi / 17 holds
        const RopePair sp = rope_pair((slot >> 1) & 7);
        const int c = slot == 16 ? 0 : (pair_slot ? ((slot & 1) ? sp.c2 : sp.c1) : slot);
        return (int)scope_token(i * kBwdQN + row, s, k_, a.mode) * row_bytes + c * 16;
    };
    auto set_dma_rows = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            qdo[j] = piece_off(i, wave + 8 * j, true);
            odo[j] = piece_off(i, wave + 8 * j, false);
        }
        if (wave < 2)
            xdo = piece_off(i, 16, wave == 0);
        else if (wave < 4)
            xdo = (int)scope_token(i * kBwdQN + opaque_lane(), s, k_, a.mode) * 4;
    };
    auto advance_dma_rows = [&](int i) __attribute__((always_inline)) {   // to tile i, from i - 1
        if constexpr (KDIV) {
            qdo[0] += tile_dn * row_bytes;
            qdo[1] += tile_dn * row_bytes;
            odo[0] += tile_dn * row_bytes;
            odo[1] += tile_dn * row_bytes;
            xdo += wave < 2 ? tile_dn * row_bytes : tile_dn * 4;
        } else {
            set_dma_rows(i);
        }
    };
    auto dma = [&](int buf) __attribute__((always_inline)) {
        char* qd = lds + buf * R::kBuf;
        char* od = qd + R::kQ;
        char* ld = od + R::kO;
        buffer_load_to_lds16(qbuf, qd + wave * 1024, qdo[0]);
        buffer_load_to_lds16(qbuf, qd + (wave + 8) * 1024, qdo[1]);
        buffer_load_to_lds16(dobuf, od + wave * 1024, odo[0]);
        buffer_load_to_lds16(dobuf, od + (wave + 8) * 1024, odo[1]);
        if (wave == 0)
            buffer_load_to_lds16(qbuf, qd + 16 * 1024, xdo);
        else if (wave == 1)
            buffer_load_to_lds16(dobuf, od + 16 * 1024, xdo);
        else if (wave == 2)
            buffer_load_to_lds4(lbuf, ld, xdo);
        else if (wave == 3)
            buffer_load_to_lds4(dlbuf, ld + 256, xdo);
    };

    const TrLane tr(lane);
    f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            dvacc[db][x] = 0.f;
            dkacc[db][x] = 0.f;
        }
    constexpr int kR1 = 2;  // depth of the operand rings: S / dP products
    constexpr int kR = 2;   // dV / dK products
    const int qb0 = 32 * qhalf;   // this wavefront's query rows in each tile
    const int nq = (a.L + kBwdQN - 1) / kBwdQN;
    set_dma_rows(0);
    dma(0);
    if (nq > 1) {
        advance_dma_rows(1);
        dma(1);
    }
    // Every load so far (the registers above and the first two tiles) has landed.  Written as
    // the compiler's own wait instruction so that it knows the register loads are complete;
    // otherwise it places its waits for them inside the loop, where they would also wait for
    // the tile loads in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt left at their maxima
    int cur = 0;   // buffer of tile i
    for (int i = 0; i < nq; ++i) {
        // this wave's pieces of tile i have landed once at most those of tile i + 1 (5 on waves
        // 0-3, 4 on the others) are outstanding
        if (i + 1 < nq) {
            if (wave < 4)
                wait_vm_loads_but<5>();
            else
                wait_vm_loads_but<4>();
        } else {
            wait_vm_loads();
        }
        __syncthreads();   // tile i is in LDS; every wavefront is done with tile i - 1
        if (i + 2 < nq) {
            advance_dma_rows(i + 2);
            dma(cur == 0 ? 2 : cur - 1);   // buffer (i + 2) mod 3 held tile i - 1
        }
        const char* qtile = lds + cur * R::kBuf;
        const char* otile = qtile + R::kQ;
        const float* ldt = reinterpret_cast<const float*>(otile + R::kO);
        cur = cur == 2 ? 0 : cur + 1;

        // start values -LSE of the queries qb0 + 8 g + 4 hf + jj this lane's accumulator rows hold
        f32x16 sacc, dpacc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(ldt + qb0 + 8 * g + 4 * hf);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                sacc[4 * g + jj] = -l4[jj];
                dpacc[4 * g + jj] = 0.f;
            }
        }
        // S = Q' K'^T and dP = dO V^T of the 32-query block: A operands from LDS, B in registers
        {
            const int r = tile_slot(qb0 + l32);
            auto qop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(qtile + r * kPitch + (2 * ks + hf) * 16);
            };
            auto oop = [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const bf16x8*>(otile + r * kPitch + (2 * ks + hf) * 16);
            };
            bf16x8 qa[kR1], oa[kR1];
#pragma unroll
            for (int ks = 0; ks < kR1 - 1; ++ks) {
                qa[ks] = qop(ks);
                oa[ks] = oop(ks);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + kR1 - 1 < KS) {
                    qa[(ks + kR1 - 1) % kR1] = qop(ks + kR1 - 1);
                    oa[(ks + kR1 - 1) % kR1] = oop(ks + kR1 - 1);
                }
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks % kR1], kreg[ks], sacc, 0, 0, 0);
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[ks % kR1], vreg[ks], dpacc, 0, 0, 0);
            }
            // Keep the S and dP products alternating, each step's two operand reads between
            // them (left alone, the compiler runs all S products and then all dP products,
            // each waiting for a read issued right after the one before it): first the four
            // log2-sum-exp reads and the ring's first reads, then per k-step an S product, a
            // read, a dP product, a read, and the last steps' products without reads.
            __builtin_amdgcn_sched_group_barrier(0x100, 4 + 2 * (kR1 - 1), 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + kR1 - 1 < KS) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
            }
        }
        // P and dZ as bf16 B operands (query qb0 + 8 g + 4 hf + jj in 16-query step g / 2, slot
        // 4 (g % 2) + jj); D is read only now, so it holds no registers during the products above
        bf16x8 pbb[2], dzb[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(ldt + kBwdQN + qb0 + 8 * g + 4 * hf);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int x = 4 * g + jj;
                const float p = __builtin_amdgcn_exp2f(sacc[x]);
                pbb[g >> 1][(g & 1) * 4 + jj] = (__bf16)p;
                dzb[g >> 1][(g & 1) * 4 + jj] = (__bf16)(p * (dpacc[x] - d4[jj]));
            }
        }
        // dV^T += dO^T P and dK^T += Q'^T dZ over the block's two 16-query steps
        {
            constexpr int NST = 2 * DB;
            auto dop = [&](int st) __attribute__((always_inline)) {
                const int kk = st / DB, db = st % DB;
                const char* ob = otile + tile_slot(qb0 + 16 * kk + tr.row) * kPitch + (4 * db + tr.gran) * 16 + tr.byte;
                return tr_operand(ob, ob + 2 * kPitch);
            };
            auto qtop = [&](int st) __attribute__((always_inline)) {
                const int kk = st / DB, db = st % DB;
                const char* qb = qtile + tile_slot(qb0 + 16 * kk + tr.row) * kPitch + (4 * db + tr.gran) * 16 + tr.byte;
                return tr_operand(qb, qb + 2 * kPitch);
            };
            bf16x8 da[kR], ka2[kR];
#pragma unroll
            for (int st = 0; st < kR - 1; ++st) {
                da[st] = dop(st);
                ka2[st] = qtop(st);
            }
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                if (st + kR - 1 < NST) {
                    da[(st + kR - 1) % kR] = dop(st + kR - 1);
                    ka2[(st + kR - 1) % kR] = qtop(st + kR - 1);
                }
                dvacc[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[st % kR], pbb[st / DB], dvacc[st % DB], 0, 0, 0);
                dkacc[st % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka2[st % kR], dzb[st / DB], dkacc[st % DB], 0, 0, 0);
            }
        }
    }

    // ---- the two query halves' partial sums meet in LDS (every load has landed, see the last wait) ----
    float* red = reinterpret_cast<float*>(lds);   // [kgrp][16 * DB values][64 lanes]
    auto exchange = [&](f32x16 (&acc)[DB]) __attribute__((always_inline)) {
        __syncthreads();
        if (qhalf == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) red[(kgrp * 16 * DB + db * 16 + x) * 64 + lane] = acc[db][x];
        }
        __syncthreads();
        if (qhalf == 0) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) acc[db][x] += red[(kgrp * 16 * DB + db * 16 + x) * 64 + lane];
        }
    };
    exchange(dvacc);
    exchange(dkacc);

    // ---- epilogue (query half 0): dv rows, and dk = (transposed RoPE of dK') / log2(e) ----
    if (qhalf != 0 || pk >= a.L) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = db * 32 + 8 * g + 4 * hf;
            const u32x2 v2 = {pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]),
                              pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(v2, dvbuf, nk * row_bytes + d0 * 2, 0, 0);
        }
    Pos kp;
    kp.t = nk / HW; kp.h = (nk / a.W) % a.H; kp.w = nk % a.W;
    store_unrotated<D, BF16>(dkacc, 0.69314718055994530942f, dkbuf, nk, row_bytes, kp, tab, a.T, a.H, a.phi_mul, lane);
}

template <int D, typename E, bool KDQ, bool KKV, bool ROT>
static hipError_t launch_bwd_k(const AttnBwdParams& a, hipStream_t stream) {
    typedef BwdLds<D> L;
    static_assert(L::kDqTab + SKIPARSE_MAX_GRID_SUM * 256 <= kLdsBytes && L::kDkvTab + SKIPARSE_MAX_GRID_SUM * 256 <= kLdsBytes &&
                  RotKvLds::kTab + SKIPARSE_MAX_GRID_SUM * 256 <= kLdsBytes, "the largest table fits LDS");
    const size_t table = (size_t)(a.T + a.H + a.W) * 256;
    const size_t lds_dq = (size_t)L::kDqTab + table, lds_kv = (size_t)L::kDkvTab + table;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, E, KDQ, ROT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dq);
    if (e != hipSuccess) return e;
    const size_t lds_kvr = (size_t)RotKvLds::kTab + table;
    if constexpr (ROT)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_rot_kernel<KKV>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_kvr);
    else
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, E, KKV>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_kv);
    if (e != hipSuccess) return e;
    // dq first: it writes D, which the dk/dv kernel reads (same stream, so in order)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, E, KDQ, ROT>), dim3(a.dq_num_work), dim3(kDqThreads), lds_dq, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (ROT)
        hipLaunchKernelGGL((attn_bwd_dkdv_rot_kernel<KKV>), dim3(a.num_work), dim3(kKvThreads), lds_kvr, stream, a);
    else
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, E, KKV>), dim3(a.num_work), dim3(kKvThreads), lds_kv, stream, a);
    return hipGetLastError();
}

template <int D, typename E, bool ROT>
static hipError_t launch_bwd_t(const AttnBwdParams& a, hipStream_t stream) {
    static_assert(kBwdQN == kBwdKN, "one divisibility test covers both tile heights");
    if (kBwdKN % a.sparse_k == 0) return launch_bwd_k<D, E, true, true, ROT>(a, stream);
    return launch_bwd_k<D, E, false, false, ROT>(a, stream);
}

hipError_t launch_attn_bwd(const AttnBwdParams& a, int head_dim, int dtype, hipStream_t stream) {
    if (head_dim == 128)
        return dtype == 0 ? launch_bwd_t<128, BF16, false>(a, stream) : launch_bwd_t<128, FP32, false>(a, stream);
    return dtype == 0 ? launch_bwd_t<64, BF16, false>(a, stream) : launch_bwd_t<64, FP32, false>(a, stream);
}

// q and k already rotated (q also scaled) by skiparse_rope_qk: head_dim 128, bf16
hipError_t launch_attn_bwd_rot(const AttnBwdParams& a, hipStream_t stream) {
    return launch_bwd_t<128, BF16, true>(a, stream);
}

int attn_bwd_block_rows() { return kBwdRows; }
int attn_bwd_dq_rows() { return kDqRows; }

}  // namespace skiparse

// Workspace of skiparse_attn_bwd_rotated_static: the backward's delta vector (rowsum of
// dout * out per (batch, head, token), fp32), written by the dq launch and read by the dk/dv
// launch of the same call.  Every GPU that loads the library holds one copy until the process
// ends; every call on that GPU shares it.  In host code the name below is only a host-side
// stand-in: its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) float scratch[skiparse::kStaticDeltaFloats];

namespace skiparse {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mutex;
float* g_static_delta[kMaxDevices] = {};
}  // namespace

hipError_t static_delta_workspace(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_static_mutex);
    if (g_static_delta[dev] == nullptr) {
        // looked up once per device, with that device current: each GPU has its own copy
        // of the array at its own address
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_static_delta[dev] = static_cast<float*>(p);
    }
    *ptr = g_static_delta[dev];
    return hipSuccess;
}

}  // namespace skiparse
