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
// wavefronts per SIMD so one wave's VALU work can fill the other's MFMA time):
//   * each wavefront owns 32 query rows and keeps Q^T for them in registers
//     as the B operand of v_mfma_f32_32x32x16_bf16;
//   * K tiles of 64 keys are staged (rotated, bf16, row-major) in LDS and are
//     the A operand, so the scores come out transposed: S^T = K Q^T.  In the
//     32x32 accumulator layout a lane then owns one query column and 16 of its
//     keys per 32-key block, so the row max is an in-lane reduction plus one
//     swap with the lane 32 away;
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
//   * K and V^T are double-buffered in LDS with padded row pitches (one extra
//     16-byte granule per row), which keeps the 16-lane access groups of both
//     the MFMA operand reads and the staging writes on distinct bank groups
//     while every LDS address stays "lane base + immediate"; the tile loop is
//     unrolled by two so the buffer index is a compile-time constant;
//   * the next tile's rows are fetched into registers before the current
//     tile's MFMAs so global latency hides behind the math;
//   * all global traffic uses buffer instructions with 32-bit offsets into the
//     (batch, head) slice; rows past the end of a scope have token indices
//     >= N, i.e. offsets past the slice, which the hardware range check turns
//     into zero loads and dropped stores;
//   * workgroup ids are remapped so the q tiles of one scope run on the same
//     XCD and share its L2 copy of the scope's K and V.
#include <type_traits>

#include "skiparse_device.hpp"
#include "skiparse_launch.hpp"

namespace skiparse {

namespace {

constexpr int kWaves = 8;                 // wavefronts per workgroup (2 per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;          // query rows per workgroup (32 per wavefront)
constexpr int kBN = 64;                   // keys per tile
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Lds {
    static constexpr int kRowPitch = D * 2 + 16;          // Q / K rows (bf16) + pad granule
    static constexpr int kVtPitch = kBN * 2 + 16;         // V^T rows (kBN bf16 slots) + pad granule
    static constexpr int kKTile = kBN * kRowPitch;
    static constexpr int kVTile = D * kVtPitch;
    static constexpr int kKOff = 0;
    static constexpr int kVOff = 2 * kKTile;
    static constexpr int kTiles = 2 * kKTile + 2 * kVTile;
    static constexpr int kQBytes = kBM * kRowPitch;       // Q staging, aliases the tiles
    static constexpr int kTabOff = kTiles > kQBytes ? kTiles : kQBytes;
};

// Key quad (keys 4*quad .. 4*quad+3 of a tile) -> its first V^T slot.  Inside
// each group of 16 keys the slot order is keys [0-3, 8-11, 4-7, 12-15]: the
// order in which the 32x32 accumulator layout hands P^T's keys to the lanes of
// a 16-deep MFMA step (lanes 0-31 hold keys {0-3, 8-11}, lanes 32-63 hold
// {4-7, 12-15}).
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

// Buffer load of NDW dwords at a byte offset.
template <int NDW>
__device__ __forceinline__ void buffer_load_dwords(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&w)[NDW]) {
    if constexpr (NDW == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = v[0]; w[1] = v[1];
    } else {
        static_assert(NDW % 4 == 0, "chunk must be a multiple of 16 bytes");
#pragma unroll
        for (int i = 0; i < NDW / 4; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
            w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    }
}

// 8 consecutive elements of E as 4 dwords of bf16 pairs (fp32 is rounded to bf16).
template <typename E>
__device__ __forceinline__ void buffer_load_8_as_bf16x2(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&w)[4]) {
    if constexpr (E::kBytes == 2) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
        w[0] = pack_bf16x2(__uint_as_float(a[0]), __uint_as_float(a[1]));
        w[1] = pack_bf16x2(__uint_as_float(a[2]), __uint_as_float(a[3]));
        w[2] = pack_bf16x2(__uint_as_float(b[0]), __uint_as_float(b[1]));
        w[3] = pack_bf16x2(__uint_as_float(b[2]), __uint_as_float(b[3]));
    }
}

// Round a rotated chunk pair to bf16 and write it to LDS at two byte addresses.
template <int CH>
__device__ __forceinline__ void store_rotated_chunks(char* a1, char* a2, const float (&x1)[CH], const float (&x2)[CH]) {
    uint32_t w1[CH / 2], w2[CH / 2];
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
        w1[i] = pack_bf16x2(x1[2 * i], x1[2 * i + 1]);
        w2[i] = pack_bf16x2(x2[2 * i], x2[2 * i + 1]);
    }
    if constexpr (CH == 8) {
        *reinterpret_cast<u32x4*>(a1) = u32x4{w1[0], w1[1], w1[2], w1[3]};
        *reinterpret_cast<u32x4*>(a2) = u32x4{w2[0], w2[1], w2[2], w2[3]};
    } else {
        *reinterpret_cast<u32x2*>(a1) = u32x2{w1[0], w1[1]};
        *reinterpret_cast<u32x2*>(a2) = u32x2{w2[0], w2[1]};
    }
}

// Grid position of a token, tracked across tiles by adding a fixed token delta
// decomposed as (dt, dh, dw) with carries.
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
    constexpr int KB = kBN / 32; // 32-key blocks of S^T
    constexpr int KK = kBN / 16; // 16-deep k-steps of P V
    constexpr int ES = E::kBytes;
    constexpr int kT = D / 8, kHW = 3 * D / 16;   // RoPE table pairs per t / h,w position
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

    build_rope_table<D>(tab, a.T, a.H, a.W);

    // This thread's RoPE chunk pair (same for its Q and K staging tasks): table rows of
    // its axis start at tbase + pos * tstride.
    const RopePair rp = rope_pair(tid & 7);
    const int tstride = rp.axis == 0 ? kT : kHW;
    const int tbase = (rp.axis == 0 ? 0 : (rp.axis == 1 ? a.T * kT : a.T * kT + a.H * kHW)) + rp.jchunk * CH;
    auto axis_pos = [&](const Pos& q) {
        // t can exceed T-1 only on rows past the end of the scope, whose data is zero
        const int t = min(q.t, a.T - 1);
        return rp.axis == 0 ? t : (rp.axis == 1 ? q.h : q.w);
    };
    auto pos_of = [&](int nn) {
        Pos q;
        q.t = nn / HW; q.h = (nn / a.W) % a.H; q.w = nn % a.W;
        return q;
    };

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
            rope_rotate<CH>(x1, x2, tab + tbase + axis_pos(pos_of(n)) * tstride);
            store_rotated_chunks<CH>(lds + r * L::kRowPitch + rp.c1 * CB, lds + r * L::kRowPitch + rp.c2 * CB, x1, x2);
        }
    }
    __syncthreads();
    bf16x8 qreg[KS];
    {
        const char* qrow = lds + (wave * 32 + l32) * L::kRowPitch + hf * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32);
    }
    __syncthreads();  // the Q area is reused by the K/V buffers below

    // ---- per-thread staging assignment ----
    // K: one (key row, RoPE chunk pair) task per thread.
    // V: one (key pair, 8-element d chunk) task per thread; lanes 0..31 of a wave take
    //    the 32 key pairs of one d chunk, so the transposed 4-byte LDS writes of 16
    //    consecutive lanes fill one V^T row segment.
    static_assert(kBN * 8 == kThreads, "one K staging task per thread");
    constexpr int VPAIRS = kBN / 2;
    constexpr int VTASKS = VPAIRS * VCH;
    static_assert(VTASKS <= kThreads, "at most one V staging task per thread");
    const int krow = tid >> 3;
    const int vpair = tid % VPAIRS;
    const int vdc = tid / VPAIRS;
    const bool v_active = VTASKS == kThreads || tid < VTASKS;
    const int vslot = key_slot_quad(vpair >> 1) + (vpair & 1) * 2;

    // loop-invariant LDS addresses (the buffer index is added as an immediate)
    const int k_rd = l32 * L::kRowPitch + hf * 16;                   // + kb*32 rows + ks*32 bytes
    const int v_rd = l32 * L::kVtPitch + hf * 16;                    // + db*32 rows + kk*32 bytes
    const int k_wr1 = krow * L::kRowPitch + rp.c1 * CB;
    const int k_wr2 = krow * L::kRowPitch + rp.c2 * CB;
    const int v_wr = 8 * vdc * L::kVtPitch + vslot * 2;              // + (2i + {0,1}) rows

    // global offsets of the staged rows, advanced per tile
    int koff1, koff2, voff[2];
    Pos kpos;
    const int tile_dn = kBN * a.sparse_k;     // token advance per tile when k | kBN
    const int dt = tile_dn / HW, rem = tile_dn % HW;
    const int dh = rem / a.W, dw = rem % a.W;
    auto set_rows = [&](int p0) {
        const int kn = (int)scope_token(p0 + krow, s, k_, a.mode);
        koff1 = kn * row_bytes + rp.c1 * CH * ES;
        koff2 = kn * row_bytes + rp.c2 * CH * ES;
        kpos = pos_of(kn);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            voff[e] = (int)scope_token(p0 + 2 * vpair + e, s, k_, a.mode) * row_bytes + vdc * 8 * ES;
    };
    set_rows(0);
    auto advance_rows = [&](int tile) {
        if (a.k_divides_bn) {
            // n(p + kBN) = n(p) + kBN*k in both modes when k divides kBN
            const int db_ = tile_dn * row_bytes;
            koff1 += db_;
            koff2 += db_;
            voff[0] += db_;
            voff[1] += db_;
            int w = kpos.w + dw, c = w >= a.W;
            kpos.w = w - (c ? a.W : 0);
            int h = kpos.h + dh + c;
            c = h >= a.H;
            kpos.h = h - (c ? a.H : 0);
            kpos.t += dt + c;
        } else {
            set_rows(tile * kBN);
        }
    };

    ChunkRaw<E, CH> kraw[2];
    uint32_t vraw[2][4];
    auto load_tile = [&]() {
        buffer_load_dwords(kbuf, koff1, kraw[0].w);
        buffer_load_dwords(kbuf, koff2, kraw[1].w);
        if (v_active) {
            buffer_load_8_as_bf16x2<E>(vbuf, voff[0], vraw[0]);
            buffer_load_8_as_bf16x2<E>(vbuf, voff[1], vraw[1]);
        }
    };

    auto store_tile = [&](auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        char* kdst = lds + L::kKOff + buf * L::kKTile;
        float x1[CH], x2[CH];
        raw_to_f32(kraw[0], x1);
        raw_to_f32(kraw[1], x2);
        rope_rotate<CH>(x1, x2, tab + tbase + axis_pos(kpos) * tstride);
        store_rotated_chunks<CH>(kdst + k_wr1, kdst + k_wr2, x1, x2);
        if (v_active) {
            char* vdst = lds + L::kVOff + buf * L::kVTile + v_wr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // dword i of each key row holds d = 8*vdc + 2i (low half) and + 2i + 1 (high half)
                const uint32_t lo = __builtin_amdgcn_perm(vraw[1][i], vraw[0][i], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(vraw[1][i], vraw[0][i], 0x07060302u);
                *reinterpret_cast<uint32_t*>(vdst + (2 * i) * L::kVtPitch) = lo;
                *reinterpret_cast<uint32_t*>(vdst + (2 * i + 1) * L::kVtPitch) = hi;
            }
        }
    };

    // ---- main loop over key tiles ----
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
    float m_run = -__builtin_inff(), l_part = 0.f;
    const float c = a.scale_log2;
    const int nt = (a.L + kBN - 1) / kBN;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    load_tile();
    store_tile(std::integral_constant<int, 0>{});
    __syncthreads();

    auto tile_step = [&](auto bufc, int j) {
        constexpr int cur = decltype(bufc)::value;
        const bool has_next = j + 1 < nt;
        if (has_next) {
            advance_rows(j + 1);
            load_tile();
        }
        const char* kcur = lds + L::kKOff + cur * L::kKTile + k_rd;
        const char* vcur = lds + L::kVOff + cur * L::kVTile + v_rd;

        // S^T = K Q^T, operand reads kept one k-step ahead of the MFMAs that consume them
        f32x16 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[kb][x] = 0.f;
        bf16x8 ka[2][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) ka[0][kb] = *reinterpret_cast<const bf16x8*>(kcur + kb * 32 * L::kRowPitch);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    ka[(ks + 1) & 1][kb] =
                        *reinterpret_cast<const bf16x8*>(kcur + kb * 32 * L::kRowPitch + (ks + 1) * 32);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks & 1][kb], qreg[ks], sacc[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 0);
#pragma unroll
        for (int i = 0; i < KS - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, KB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KB, 0);
        __builtin_amdgcn_s_setprio(0);

        // keys past the end of the scope (last tile only)
        if (j == nt - 1 && (a.L % kBN) != 0) {
            const int valid = a.L - j * kBN;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (kb * 32 + 8 * g + 4 * hf + jj >= valid) sacc[kb][4 * g + jj] = -__builtin_inff();
        }

        // online softmax: tile max per query (in-lane, then across the two lane halves)
        float mt = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mt = fmaxf(mt, sacc[kb][x]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float mnew = fmaxf(m_run, mt);
        if (__ballot((mnew - m_run) * c > kRescaleLog2) != 0ull) {
            const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * c);
            m_run = mnew;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) o[db][x] *= alpha;
        }
        bf16x8 pb[KK];
        {
            const float mc = m_run * c;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    // keys 32kb + 8g + 4hf + jj sit in k-step 2kb + g/2, slots (g%2)*4 + jj
                    const int kk = 2 * kb + (g >> 1), sl = (g & 1) * 4;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        pb[kk][sl + jj] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][4 * g + jj], c, -mc));
                }
            float lsum = l_part;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const bf16x2 pair = {pb[kk][2 * x], pb[kk][2 * x + 1]};
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lsum, false);
                }
            l_part = lsum;
        }

        // O^T += V^T P^T, V operands read one k-step ahead
        bf16x8 va[2][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) va[0][db] = *reinterpret_cast<const bf16x8*>(vcur + db * 32 * L::kVtPitch);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 1 < KK) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    va[(kk + 1) & 1][db] =
                        *reinterpret_cast<const bf16x8*>(vcur + db * 32 * L::kVtPitch + (kk + 1) * 32);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk & 1][db], pb[kk], o[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
#pragma unroll
        for (int i = 0; i < KK - 1; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, DB, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
        __builtin_amdgcn_s_setprio(0);

        if (has_next) store_tile(std::integral_constant<int, cur ^ 1>{});
        __syncthreads();
    };

    for (int j = 0; j < nt; j += 2) {
        tile_step(std::integral_constant<int, 0>{}, j);
        if (j + 1 < nt) tile_step(std::integral_constant<int, 1>{}, j + 1);
    }

    // ---- epilogue: normalise and scatter rows back to their tokens ----
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
        const float inv = 1.0f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
        const int p = qt * kBM + wave * 32 + l32;
        const int off = (int)scope_token(p, s, k_, a.mode) * row_bytes;   // past the slice when p >= L
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
