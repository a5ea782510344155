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
// Tiling (one workgroup = 8 wavefronts = 256 query rows of one scope; two
// wavefronts per SIMD so one wave's softmax VALU work overlaps the other's
// MFMAs):
//   * each wavefront owns 32 query rows and keeps Q^T for them in registers
//     as the B operand of v_mfma_f32_32x32x16_bf16;
//   * K tiles of 64 keys are staged (rotated, bf16, row-major, XOR-swizzled)
//     in LDS and are the A operand, so the scores come out transposed:
//     S^T = K Q^T.  In the 32x32 accumulator layout a lane then owns one query
//     column and 16 of its keys per 32-key block, so the row max is an in-lane
//     reduction plus one swap with the lane 32 away;
//   * P^T (bf16) is fed to O^T += V^T P^T straight from the accumulator
//     registers as the B operand.  The MFMA contracts over whatever key order
//     the operand slots carry, so V is staged transposed in LDS with its keys
//     in exactly the slot order in which P^T's accumulator layout holds them;
//   * online softmax in fp32 with exp2 and log2(e)/sqrt(d) folded into one FMA;
//     the row sum is accumulated from the bf16 P pairs with a 2-way dot
//     instruction, so it sums exactly the weights the PV product uses.  The
//     running maximum is only moved when a tile raises it by more than 2^8 in
//     the exponent (the result is identical up to rounding, since the same
//     maximum is used for numerator and denominator), which skips most
//     rescales of the O^T accumulator;
//   * K and V^T are double-buffered in LDS; the next tile's rows are fetched
//     into registers before the current tile's MFMAs so global latency hides
//     behind the math;
//   * workgroup ids are remapped so the q tiles of one scope run on the same
//     XCD and share its L2 copy of the scope's K and V.
#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

namespace {

constexpr int kWaves = 8;                 // wavefronts per workgroup (2 per SIMD)
constexpr int kQB = 1;                    // 32-query blocks per wavefront
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kQB * kWaves;    // query rows per workgroup
constexpr int kBN = 64;                   // keys per tile
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Lds {
    static constexpr int kKTile = kBN * D * 2;         // bf16 K tile
    static constexpr int kVTile = D * kBN * 2;         // bf16 V^T tile
    static constexpr int kKOff = 0;
    static constexpr int kVOff = 2 * kKTile;
    static constexpr int kTiles = 2 * kKTile + 2 * kVTile;
    static constexpr int kQBytes = kBM * D * 2;        // Q staging, aliases the tiles
    static constexpr int kTabOff = kTiles > kQBytes ? kTiles : kQBytes;
};

// Row-major bf16 rows of D elements (Q and K), 16-byte granules XOR-swizzled
// by the row index so that 16 lanes reading one granule column of 16
// consecutive rows hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int row_addr(int row, int byte_in_row) {
    constexpr int G = D / 8;
    return row * (D * 2) + ((((byte_in_row >> 4) ^ (row & (G - 1)))) << 4) + (byte_in_row & 15);
}

// V^T rows: one row of kBN key slots (2*kBN bytes) per head-dim index d.  The
// 16-byte granule index is XOR-swizzled with bits of d so that both access
// patterns spread over the bank groups of a 256-byte line: 16 consecutive d
// rows read at one granule column (the MFMA operand reads) hit 16 different
// groups, and the staging writes of one key quad to rows d = 8c + 2i for 16
// consecutive c hit each group at most twice.
__device__ __forceinline__ int vt_addr(int d, int slot) {
    constexpr int VG = kBN / 8;       // granules per V^T row
    constexpr int RPL = 128 / kBN;    // V^T rows per 256-byte line
    const int f = ((d / RPL) ^ (d / (RPL * VG))) & (VG - 1);
    return d * (kBN * 2) + (((slot >> 3) ^ f) << 4) + ((slot & 7) << 1);
}

// Key quad (keys 4*quad .. 4*quad+3 of a tile) -> its first V^T slot.  Inside each group of 16 keys the
// slot order is keys [0-3, 8-11, 4-7, 12-15]: the order in which the 32x32
// accumulator layout hands P^T's keys to the lanes of a 16-deep MFMA step
// (lanes 0-31 hold keys {0-3, 8-11}, lanes 32-63 hold {4-7, 12-15}).
__device__ __forceinline__ int key_slot_quad(int quad) {
    const int m = quad & 3;
    return (quad >> 2) * 16 + ((((m & 1) << 1) | (m >> 1)) << 2);
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int q8 = nblocks >> 3, r8 = nblocks & 7;
    const int xcd = bid & 7, slot = bid >> 3;
    return xcd * q8 + min(xcd, r8) + slot;
}

// Raw element storage of one RoPE chunk (CH elements of E) as dwords.
template <typename E, int CH>
struct ChunkRaw {
    static constexpr int kDwords = CH * E::kBytes / 4;
    uint32_t w[kDwords];
};

template <int NDW>
__device__ __forceinline__ void load_dwords(const void* p, uint32_t (&w)[NDW]) {
    if constexpr (NDW == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(p);
        w[0] = v[0]; w[1] = v[1];
    } else {
        static_assert(NDW % 4 == 0, "chunk must be a multiple of 16 bytes");
#pragma unroll
        for (int i = 0; i < NDW / 4; ++i) {
            const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
            w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    }
}

template <typename E, int CH>
__device__ __forceinline__ void raw_to_f32(const ChunkRaw<E, CH>& r, float (&x)[CH]) {
    if constexpr (E::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < CH / 2; ++i) {
            x[2 * i] = __uint_as_float(r.w[i] << 16);
            x[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < CH; ++i) x[i] = __uint_as_float(r.w[i]);
    }
}

// Raw element storage of 8 consecutive elements of E, as 4 dwords of bf16 pairs.
template <typename E>
__device__ __forceinline__ void load_8_as_bf16x2(const void* p, uint32_t (&w)[4]) {
    if constexpr (E::kBytes == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
        const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
        const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
        w[0] = pack_bf16x2(a[0], a[1]); w[1] = pack_bf16x2(a[2], a[3]);
        w[2] = pack_bf16x2(b[0], b[1]); w[3] = pack_bf16x2(b[2], b[3]);
    }
}

struct Pos {
    int t, h, w;
};

}  // namespace

template <int D, typename E>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kThreads / 256, kThreads / 256)))
attn_fwd_kernel(AttnParams a) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    typedef Lds<D> L;
    constexpr int CH = D / 16;   // elements per RoPE chunk
    constexpr int CB = CH * 2;   // bytes per RoPE chunk in LDS (bf16)
    constexpr int KS = D / 16;   // 16-deep k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    constexpr int VCH = D / 8;   // 8-element d-chunks per V row
    float2* tab = reinterpret_cast<float2*>(lds + L::kTabOff);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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
    const int64_t row_stride = (int64_t)a.heads * D;                      // elements per token
    const int64_t batch_head_off = (int64_t)b * a.N * row_stride + (int64_t)head * D;
    const int HW = a.H * a.W;

    build_rope_table<D>(tab, a.T, a.H, a.W);

    // ---- stage the Q tile (rotated) into LDS, then into registers ----
    {
        const int p0 = qt * kBM;
        const int cp = tid & 7;
        const RopePair rp = rope_pair(cp);
        __syncthreads();  // table ready
#pragma unroll 2
        for (int it = 0; it < kBM * 8 / kThreads; ++it) {
            const int r = (tid >> 3) + it * (kThreads / 8);
            const int p = p0 + r;
            float x1[CH], x2[CH];
            if (p < a.L) {
                const int64_t n = scope_token(p, s, k_, a.mode);
                const char* src = reinterpret_cast<const char*>(a.q) +
                                  (batch_head_off + n * row_stride) * E::kBytes;
                ChunkRaw<E, CH> r1, r2;
                load_dwords(src + rp.c1 * CH * E::kBytes, r1.w);
                load_dwords(src + rp.c2 * CH * E::kBytes, r2.w);
                raw_to_f32(r1, x1);
                raw_to_f32(r2, x2);
                const int nn = (int)n;
                const int pos = rp.axis == 0 ? nn / HW : (rp.axis == 1 ? (nn / a.W) % a.H : nn % a.W);
                rope_rotate<CH>(x1, x2, tab + rope_row<D>(rp.axis, pos, a.T, a.H) + rp.jchunk * CH);
            } else {
#pragma unroll
                for (int e = 0; e < CH; ++e) { x1[e] = 0.f; x2[e] = 0.f; }
            }
            uint32_t w1[CH / 2], w2[CH / 2];
#pragma unroll
            for (int i = 0; i < CH / 2; ++i) {
                w1[i] = pack_bf16x2(x1[2 * i], x1[2 * i + 1]);
                w2[i] = pack_bf16x2(x2[2 * i], x2[2 * i + 1]);
            }
            if constexpr (CH == 8) {
                *reinterpret_cast<u32x4*>(lds + row_addr<D>(r, rp.c1 * CB)) = u32x4{w1[0], w1[1], w1[2], w1[3]};
                *reinterpret_cast<u32x4*>(lds + row_addr<D>(r, rp.c2 * CB)) = u32x4{w2[0], w2[1], w2[2], w2[3]};
            } else {
                *reinterpret_cast<u32x2*>(lds + row_addr<D>(r, rp.c1 * CB)) = u32x2{w1[0], w1[1]};
                *reinterpret_cast<u32x2*>(lds + row_addr<D>(r, rp.c2 * CB)) = u32x2{w2[0], w2[1]};
            }
        }
    }
    __syncthreads();
    bf16x8 qreg[kQB][KS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = (wave * kQB + qb) * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[qb][ks] = *reinterpret_cast<const bf16x8*>(lds + row_addr<D>(row, (2 * ks + hf) * 16));
    }
    __syncthreads();  // the Q area is reused by the K/V buffers below

    // ---- per-thread staging assignment: NKR key rows (K) and one key quad (V) ----
    constexpr int NKR = kBN * 8 / kThreads;   // K rows staged per thread per tile
    constexpr int KB = kBN / 32;              // 32-key blocks of S^T
    constexpr int KK = kBN / 16;              // 16-deep k-steps of P V
    const int kcp = tid & 7;
    const RopePair krp = rope_pair(kcp);
    const int vquad = tid / VCH;              // keys 4*vquad .. 4*vquad+3
    const int vdc = tid % VCH;                // d = 8*vdc .. 8*vdc+7
    const bool v_active = tid < (kBN / 4) * VCH;
    const int vslot = key_slot_quad(vquad & (kBN / 4 - 1));
    auto krow = [&](int i) { return (tid >> 3) + i * (kThreads / 8); };

    // token index and grid position of each staged key row, advanced per tile
    int kn[NKR];
    Pos kpos[NKR];
    int vn[4];
    const int tile_dn = kBN * a.sparse_k;     // token advance per tile when k | kBN
    const int dt = tile_dn / HW, rem = tile_dn % HW;
    const int dh = rem / a.W, dw = rem % a.W;
    auto pos_of = [&](int nn) {
        Pos q;
        q.t = nn / HW; q.h = (nn / a.W) % a.H; q.w = nn % a.W;
        return q;
    };
#pragma unroll
    for (int i = 0; i < NKR; ++i) {
        kn[i] = (int)scope_token(krow(i), s, k_, a.mode);
        kpos[i] = pos_of(kn[i]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vn[e] = (int)scope_token(4 * vquad + e, s, k_, a.mode);

    auto advance_rows = [&](int tile) {
        if (a.k_divides_bn) {
            // n(p + kBN) = n(p) + kBN*k in both modes when k divides kBN
#pragma unroll
            for (int i = 0; i < NKR; ++i) {
                kn[i] += tile_dn;
                int w = kpos[i].w + dw, c = w >= a.W;
                kpos[i].w = w - (c ? a.W : 0);
                int h = kpos[i].h + dh + c;
                c = h >= a.H;
                kpos[i].h = h - (c ? a.H : 0);
                kpos[i].t += dt + c;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) vn[e] += tile_dn;
        } else {
            const int p0 = tile * kBN;
#pragma unroll
            for (int i = 0; i < NKR; ++i) {
                kn[i] = (int)scope_token(p0 + krow(i), s, k_, a.mode);
                kpos[i] = pos_of(kn[i]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) vn[e] = (int)scope_token(p0 + 4 * vquad + e, s, k_, a.mode);
        }
    };

    ChunkRaw<E, CH> kraw[NKR][2];
    uint32_t vraw[4][4];
    const char* kbase = reinterpret_cast<const char*>(a.k) + batch_head_off * E::kBytes;
    const char* vbase = reinterpret_cast<const char*>(a.v) + batch_head_off * E::kBytes;

    auto load_tile = [&](int tile) {
        const int p0 = tile * kBN;
#pragma unroll
        for (int i = 0; i < NKR; ++i) {
            if (p0 + krow(i) < a.L) {
                const char* src = kbase + (int64_t)kn[i] * row_stride * E::kBytes;
                load_dwords(src + krp.c1 * CH * E::kBytes, kraw[i][0].w);
                load_dwords(src + krp.c2 * CH * E::kBytes, kraw[i][1].w);
            } else {
#pragma unroll
                for (int x = 0; x < ChunkRaw<E, CH>::kDwords; ++x) { kraw[i][0].w[x] = 0u; kraw[i][1].w[x] = 0u; }
            }
        }
        if (v_active) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (p0 + 4 * vquad + e < a.L) {
                    load_8_as_bf16x2<E>(vbase + ((int64_t)vn[e] * row_stride + vdc * 8) * E::kBytes, vraw[e]);
                } else {
                    vraw[e][0] = vraw[e][1] = vraw[e][2] = vraw[e][3] = 0u;
                }
            }
        }
    };

    auto store_tile = [&](int buf, int tile) {
        char* kdst = lds + L::kKOff + buf * L::kKTile;
#pragma unroll
        for (int i = 0; i < NKR; ++i) {
            float x1[CH], x2[CH];
            raw_to_f32(kraw[i][0], x1);
            raw_to_f32(kraw[i][1], x2);
            // rows past the end of the scope hold zeros; their (out-of-grid) position is not looked up
            const bool valid = tile * kBN + krow(i) < a.L;
            const int pos = !valid ? 0 : (krp.axis == 0 ? kpos[i].t : (krp.axis == 1 ? kpos[i].h : kpos[i].w));
            rope_rotate<CH>(x1, x2, tab + rope_row<D>(krp.axis, pos, a.T, a.H) + krp.jchunk * CH);
            uint32_t w1[CH / 2], w2[CH / 2];
#pragma unroll
            for (int j = 0; j < CH / 2; ++j) {
                w1[j] = pack_bf16x2(x1[2 * j], x1[2 * j + 1]);
                w2[j] = pack_bf16x2(x2[2 * j], x2[2 * j + 1]);
            }
            if constexpr (CH == 8) {
                *reinterpret_cast<u32x4*>(kdst + row_addr<D>(krow(i), krp.c1 * CB)) = u32x4{w1[0], w1[1], w1[2], w1[3]};
                *reinterpret_cast<u32x4*>(kdst + row_addr<D>(krow(i), krp.c2 * CB)) = u32x4{w2[0], w2[1], w2[2], w2[3]};
            } else {
                *reinterpret_cast<u32x2*>(kdst + row_addr<D>(krow(i), krp.c1 * CB)) = u32x2{w1[0], w1[1]};
                *reinterpret_cast<u32x2*>(kdst + row_addr<D>(krow(i), krp.c2 * CB)) = u32x2{w2[0], w2[1]};
            }
        }
        if (v_active) {
            char* vdst = lds + L::kVOff + buf * L::kVTile;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // dword i of each key row holds d = 8*vdc + 2i (low half) and + 2i + 1 (high half)
                const uint32_t lo01 = __builtin_amdgcn_perm(vraw[1][i], vraw[0][i], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(vraw[3][i], vraw[2][i], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(vraw[1][i], vraw[0][i], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(vraw[3][i], vraw[2][i], 0x07060302u);
                const int d = 8 * vdc + 2 * i;
                *reinterpret_cast<u32x2*>(vdst + vt_addr(d, vslot)) = u32x2{lo01, lo23};
                *reinterpret_cast<u32x2*>(vdst + vt_addr(d + 1, vslot)) = u32x2{hi01, hi23};
            }
        }
    };

    // ---- main loop over key tiles ----
    f32x16 o[DB][kQB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int x = 0; x < 16; ++x) o[db][qb][x] = 0.f;
    float m_run[kQB], l_part[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m_run[qb] = -__builtin_inff();
        l_part[qb] = 0.f;
    }
    const float c = a.scale_log2;
    const int nt = (a.L + kBN - 1) / kBN;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    load_tile(0);
    store_tile(0, 0);
    __syncthreads();

    for (int j = 0; j < nt; ++j) {
        const int cur = j & 1;
        const bool has_next = j + 1 < nt;
        if (has_next) {
            advance_rows(j + 1);
            load_tile(j + 1);
        }
        const char* kcur = lds + L::kKOff + cur * L::kKTile;
        const char* vcur = lds + L::kVOff + cur * L::kVTile;

        // S^T = K Q^T
        f32x16 sacc[KB][kQB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                for (int x = 0; x < 16; ++x) sacc[kb][qb][x] = 0.f;
        bf16x8 ka[2][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            ka[0][kb] = *reinterpret_cast<const bf16x8*>(kcur + row_addr<D>(kb * 32 + l32, hf * 16));
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    ka[(ks + 1) & 1][kb] = *reinterpret_cast<const bf16x8*>(
                        kcur + row_addr<D>(kb * 32 + l32, (2 * (ks + 1) + hf) * 16));
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
                    sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1][kb], qreg[qb][ks], sacc[kb][qb], 0, 0, 0);
        }
        // keep the operand reads one k-step ahead of the MFMAs that consume them
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 0);
#pragma unroll
        for (int i = 0; i < KS - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, KB * kQB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KB * kQB, 0);
        __builtin_amdgcn_s_setprio(0);

        // keys past the end of the scope (last tile only)
        if (j == nt - 1 && (a.L % kBN) != 0) {
            const int valid = a.L - j * kBN;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int key = kb * 32 + 8 * g + 4 * hf + jj;
                        if (key >= valid) {
#pragma unroll
                            for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb][4 * g + jj] = -__builtin_inff();
                        }
                    }
        }

        // online softmax: tile max per query (in-lane, then across the two lane halves)
        float mnew[kQB];
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            float mt = sacc[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int x = 0; x < 16; ++x) mt = fmaxf(mt, sacc[kb][qb][x]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            mnew[qb] = fmaxf(m_run[qb], mt);
            need |= (mnew[qb] - m_run[qb]) * c > kRescaleLog2;
        }
        if (__ballot(need) != 0ull) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - mnew[qb]) * c);
                m_run[qb] = mnew[qb];
                l_part[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int x = 0; x < 16; ++x) o[db][qb][x] *= alpha;
            }
        }
        bf16x8 pb[kQB][KK];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const float mc = m_run[qb] * c;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // keys 32kb + 8g + 4hf + jj sit in k-step 2kb + g/2, slots (g%2)*4 + jj
                    const int kk = 2 * kb + (g >> 1), sl = (g & 1) * 4;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        pb[qb][kk][sl + jj] =
                            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][4 * g + jj], c, -mc));
                }
            float lsum = l_part[qb];
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const bf16x2 pair = {pb[qb][kk][2 * x], pb[qb][kk][2 * x + 1]};
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lsum, false);
                }
            l_part[qb] = lsum;
        }

        // O^T += V^T P^T, V operands prefetched one step ahead
        bf16x8 va[2][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
            va[0][db] = *reinterpret_cast<const bf16x8*>(vcur + vt_addr(db * 32 + l32, hf * 8));
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 1 < KK) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    va[(kk + 1) & 1][db] = *reinterpret_cast<const bf16x8*>(
                        vcur + vt_addr(db * 32 + l32, (kk + 1) * 16 + hf * 8));
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
                    o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk & 1][db], pb[qb][kk], o[db][qb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
#pragma unroll
        for (int i = 0; i < KK - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, DB * kQB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, DB, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DB * kQB, 0);
        __builtin_amdgcn_s_setprio(0);

        if (has_next) store_tile(cur ^ 1, j + 1);
        __syncthreads();
    }

    // ---- epilogue: normalise and scatter rows back to their tokens ----
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[qb]), __float_as_uint(l_part[qb]),
                                                         false, false);
        const float lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / lsum;
        const int p = qt * kBM + (wave * kQB + qb) * 32 + l32;
        if (p < a.L) {
            const int64_t n = scope_token(p, s, k_, a.mode);
            char* dst = reinterpret_cast<char*>(a.out) + (batch_head_off + n * row_stride) * E::kBytes;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + 8 * g + 4 * hf;
                    const float y0 = o[db][qb][4 * g] * inv, y1 = o[db][qb][4 * g + 1] * inv;
                    const float y2 = o[db][qb][4 * g + 2] * inv, y3 = o[db][qb][4 * g + 3] * inv;
                    if constexpr (E::kBytes == 2) {
                        *reinterpret_cast<u32x2*>(dst + d0 * 2) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                    } else {
                        *reinterpret_cast<f32x4*>(dst + d0 * 4) = f32x4{y0, y1, y2, y3};
                    }
                }
        }
    }
}

template <int D, typename E>
static hipError_t launch_attn_t(const AttnParams& a, hipStream_t stream) {
    typedef Lds<D> L;
    const size_t lds = (size_t)L::kTabOff + (size_t)rope_table_pairs(a.T, a.H, a.W, D) * sizeof(float2);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<D, E>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_fwd_kernel<D, E>), dim3(a.num_work), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnParams& a, int head_dim, int dtype, hipStream_t stream) {
    if (head_dim == 128) return dtype == 0 ? launch_attn_t<128, BF16>(a, stream) : launch_attn_t<128, FP32>(a, stream);
    return dtype == 0 ? launch_attn_t<64, BF16>(a, stream) : launch_attn_t<64, FP32>(a, stream);
}

int attn_block_rows() { return kBM; }
int attn_tile_keys() { return kBN; }

}  // namespace skiparse
