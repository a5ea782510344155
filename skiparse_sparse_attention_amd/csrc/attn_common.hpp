// Device helpers shared by the Skiparse attention kernels (forward and backward): the
// banked 3D-RoPE table in LDS, XCD-aware workgroup numbering, RoPE chunk handling, buffer
// loads and stores, loads into LDS, waits, and the LDS transpose read.
#pragma once

#include "skiparse_device.hpp"

namespace skiparse {
namespace attn {

// Q and K rows in LDS hold RoPE chunk pair cp (first-half chunk c1, partner c2) in chunk slots
// 2 cp and 2 cp + 1, i.e. each rotate-half pair in one 32-byte span (Q and K use the same order,
// and Q K^T contracts over head_dim in any order).  With the one-granule row pad, granule g of
// row r falls in bank group (r + g) mod 16 (D = 128): the MFMA operand reads (one granule of 16
// consecutive rows per 16 lanes) are conflict-free, and so are the staging writes of a 16-lane
// group (two consecutive rows times eight pairs), whose first store covers the even slots and
// whose second store covers the odd ones.

// 3D-RoPE (cos, sin) table of the attention kernel: one 256-byte row per axis position
// (T t rows, then H h rows, then W w rows); pair j of a row sits at byte 16*off + 8*j.
// Each staging group of 16 lanes covers two consecutive key rows times the eight chunk
// pairs, and in instruction i the lanes of one axis read granules off + i + m*CH/2.  The
// offsets put t, h and the w rows of even and odd "phi" into different granule classes, so
// those reads never share a bank whenever the two rows share their t and h positions (the
// common case): t at 0, h at 1 (D = 128) or 4 (D = 64), w at 2 + phi or 9 + phi, where phi
// is the parity of w div phi_div -- phi_div being the w step between consecutive rows of a
// scope (k for Single Skip, 1 for Group Skip).  phi only moves data, never changes values.
template <int D>
struct RopeBank {
    static constexpr int kOffH = D == 128 ? 1 : 4;
    static constexpr int kOffW = D == 128 ? 2 : 9;
    static_assert(D == 64 || D == 128, "head_dim");
};

// V rows in LDS: granule g of row r is stored at granule g ^ vswz(r).  The PV operand reads
// (ds_read_b64_tr_b16) fetch, per 32 lanes, the same four-granule block of four consecutive
// rows; vswz moves those rows' blocks apart (by r mod 4 at D = 128; at D = 64 the row parity
// already separates rows r and r + 1 and vswz separates r and r + 2), so the 32 lanes hit
// distinct banks.  Rows are written whole by 64-lane 1 KiB loads, conflict-free in any order.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return (r & 3) << 2;
    else return ((r >> 1) & 1) << 2;
}

__device__ __forceinline__ int rope_phi(int w, int phi_mul) { return ((w * phi_mul) >> 16) & 1; }

template <int D>
__device__ __forceinline__ void build_banked_rope_table(char* tab, int T, int H, int W, int phi_mul) {
    constexpr int kT = D / 8;        // pairs per t position
    constexpr int kHW = 3 * D / 16;  // pairs per h or w position
    const int tid = threadIdx.x, nthr = blockDim.x;   // nthr: a multiple of kT
    auto put = [&](int off, int j, int pos, double inv_freq) __attribute__((always_inline)) {
        const double theta = (double)pos * inv_freq;
        double sn, cs;
        sincos(theta, &sn, &cs);
        *reinterpret_cast<float2*>(tab + off + 8 * j) = make_float2((float)cs, (float)sn);
    };
    // Each thread keeps one pair index per axis, so it evaluates the float64 frequency
    // 10000^(-2j/d_a) once per axis instead of once per table entry (same expressions, same
    // values).  t axis: pair tid % kT of positions tid / kT, tid / kT + nthr / kT, ...
    {
        const int j = tid % kT;
        const double inv_freq = pow(10000.0, -2.0 * (double)j / (double)(D / 4));
        for (int pos = tid / kT; pos < T; pos += nthr / kT) put(pos * 256, j, pos, inv_freq);
    }
    // h and w axes share their frequencies: pair tid % kHW, for the threads of whole groups of kHW
    const int groups = nthr / kHW;
    if (tid < groups * kHW) {
        const int j = tid % kHW;
        const double inv_freq = pow(10000.0, -2.0 * (double)j / (double)(3 * D / 8));
        for (int pos = tid / kHW; pos < H; pos += groups) put((T + pos) * 256 + RopeBank<D>::kOffH * 16, j, pos, inv_freq);
        for (int pos = tid / kHW; pos < W; pos += groups)
            put((T + H + pos) * 256 + (RopeBank<D>::kOffW + rope_phi(pos, phi_mul)) * 16, j, pos, inv_freq);
    }
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

// Rotate-half pair rotation with table entries preloaded as f32x4 = two (cos, sin) pairs.
template <int CH>
__device__ __forceinline__ void rope_rotate_cs(float (&x1)[CH], float (&x2)[CH], const f32x4 (&cs)[CH / 2]) {
#pragma unroll
    for (int e = 0; e < CH; ++e) {
        const float c = cs[e / 2][2 * (e % 2)], sn = cs[e / 2][2 * (e % 2) + 1];
        const float a = x1[e], b = x2[e];
        x1[e] = a * c - b * sn;
        x2[e] = b * c + a * sn;
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

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at dst + 16 l (dst
// must be wave-uniform; out-of-range offsets write zeros).  Issued as inline assembly so the
// compiler does not treat every later LDS read as a possible reader of this write and wait for
// all outstanding loads before it; the caller instead waits for the load counter (vmcnt) before
// the barrier after which the data is read.  The s_nop covers the M0-write hazard.
__device__ __forceinline__ void buffer_load_to_lds16(__amdgpu_buffer_rsrc_t r, char* dst, int off) {
    const unsigned lds_addr = (unsigned)(size_t)((__attribute__((address_space(3))) char*)dst);
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr) : "memory");
}

// Wait until every vector memory load of this wave has completed (including loads into LDS).
__device__ __forceinline__ void wait_vm_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector memory instructions of this wave are outstanding: every load
// issued before the N most recent ones has completed (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_loads_but() { asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory"); }

// LDS transpose read of 4 bf16 (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane j receives element j % 4 of the 4-element runs addressed by lanes 4t + j / 4,
// t = 0..3.
__device__ __forceinline__ i16x4 ds_read_tr16(const char* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Online softmax of one 64-key tile for the forward kernels (Open-Sora Plan documentation,
// "Skiparse Attention": softmax attention within each scope, taken tile by tile).  The wave
// holds S'^T of 64 keys x 32 queries as two 32x32 MFMA accumulators: lane l holds query
// l % 32 and, of each 32-key block kb, keys 32 kb + 8 g + 4 (l / 32) + jj in slot 4 g + jj.
// Scores arrive as S' = s log2(e)/sqrt(d) - m_ref, m_ref being the row's reference (the QK
// products start from s_init = -m_ref).  The weights are P = exp2(S'), rounded to bf16 into pb
// (k-step 2 kb + g / 2, slots (g % 2) * 4 + jj: the B operand layout of the P V product), and
// the row sum l_part gathers the unrounded fp32 weights of the lane's 32 keys (the two lane
// halves are added at the end).  The reference is lazy: it is set on the first tile to the
// tile's row max, and later moves (by the row max, if positive) only when some lane's 32
// weights sum to more than 2^8, after which the tile's weights are recomputed.  So every
// weight entering pb and l_part is at most 2^8, and O and l_part are rescaled only then.
// On a partial tile (`partial`), keys at or past `valid` are masked to -inf (weight 0).
// kPinInit: s_init is made opaque to the compiler where it is written.  Left alone, the
// compiler treats s_init as the splat of -m_ref and rebuilds its register copies after every
// tile (31 moves per tile in the rotated kernel, whose QK products read s_init in place); with
// the pin the copies are rewritten only when the reference moves (rotated kernel 1.2 % faster,
// the fused kernel 2.9 % slower with it, so only the rotated kernel sets it).
template <int DB, bool kPinInit = false>
__device__ __forceinline__ void softmax_tile(f32x16 (&sacc)[2], f32x16 (&o)[DB], bf16x8 (&pb)[4], f32x16& s_init,
                                             float& m_ref, float& l_part, bool first, bool partial, int valid,
                                             int hf) {
    constexpr float kSumLimit = 256.0f;
    if (partial) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (kb * 32 + 8 * g + 4 * hf + jj >= valid) sacc[kb][4 * g + jj] = -__builtin_inff();
    }
    // row max of the tile relative to the reference: in-lane, then across the lane halves
    auto tile_max = [&]() __attribute__((always_inline)) {
        float mt = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mt = fmaxf(mt, sacc[kb][x]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    auto move_ref = [&](float delta) __attribute__((always_inline)) {
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        m_ref += delta;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) o[db][x] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[kb][x] -= delta;
#pragma unroll
        for (int x = 0; x < 16; ++x) s_init[x] = -m_ref;
        if constexpr (kPinInit) asm volatile("" : "+v"(s_init));
    };
    // weights into pb; returns the lane's sum of its 32 unrounded weights (four chains)
    auto weights = [&]() __attribute__((always_inline)) {
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int kk = 2 * kb + (g >> 1), sl = (g & 1) * 4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float e = __builtin_amdgcn_exp2f(sacc[kb][4 * g + jj]);
                    pb[kk][sl + jj] = (__bf16)e;
                    ls[jj] += e;
                }
            }
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    if (first) {
        // O and l_part are still zero: only the reference moves.  (Scaling them by
        // exp2(-max) would turn 0 into NaN when a row's first-tile scores all lie below -128.)
        const float mt = tile_max();
        m_ref += mt;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) sacc[kb][x] -= mt;
#pragma unroll
        for (int x = 0; x < 16; ++x) s_init[x] = -m_ref;
        if constexpr (kPinInit) asm volatile("" : "+v"(s_init));
    }
    float hs = weights();
    if (__ballot(hs > kSumLimit) != 0ull) {
        move_ref(fmaxf(tile_max(), 0.f));
        hs = weights();
    }
    l_part += hs;
}

// Grid position of a token, tracked across tiles by adding a fixed token delta
// decomposed as (dt, dh, dw) with carries.
struct Pos {
    int t, h, w;
};


// Byte offset, in the banked table, of the (cos, sin) entry of pair j of `axis` (0 = t, 1 = h,
// 2 = w) at grid position pos (j counts the axis' rotate-half pairs from 0).
template <int D>
__device__ __forceinline__ int rope_tab_offset(int T, int H, int axis, int pos, int j, int phi_mul) {
    const int row = axis == 0 ? pos * 256
                  : axis == 1 ? (T + pos) * 256 + RopeBank<D>::kOffH * 16
                              : (T + H + pos) * 256 + (RopeBank<D>::kOffW + rope_phi(pos, phi_mul)) * 16;
    return row + 8 * j;
}

// One (row, RoPE chunk pair) staging task: the pair's two chunks of the token at byte offset
// `off` (chunk c at off + c*CH*E bytes) rotated by 3D RoPE at grid position q, multiplied by
// `scale`, rounded to bf16 and written into an LDS row in the pair-slot order (slots 2 cp and
// 2 cp + 1).  Out-of-range offsets load zeros.
template <int D, typename E>
__device__ __forceinline__ void stage_rotated_pair(__amdgpu_buffer_rsrc_t r, int off, const RopePair& rp, int cp,
                                                   const char* tab, int T, int H, const Pos& q, int phi_mul,
                                                   float scale, char* lds_row) {
    constexpr int CH = D / 16;
    constexpr int ES = E::kBytes;
    ChunkRaw<E, CH> r1, r2;
    buffer_load_dwords(r, off + rp.c1 * CH * ES, r1.w);
    buffer_load_dwords(r, off + rp.c2 * CH * ES, r2.w);
    float x1[CH], x2[CH];
    raw_to_f32(r1, x1);
    raw_to_f32(r2, x2);
    // t can exceed T-1 only on rows past the end of a scope, whose data is zero
    const int pos = rp.axis == 0 ? min(q.t, T - 1) : (rp.axis == 1 ? q.h : q.w);
    const char* row = tab + rope_tab_offset<D>(T, H, rp.axis, pos, rp.jchunk * CH, rp.axis == 2 ? phi_mul : 0);
    f32x4 cs[CH / 2];
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) cs[i] = *reinterpret_cast<const f32x4*>(row + 16 * i);
    rope_rotate_cs<CH>(x1, x2, cs);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
        x1[e] *= scale;
        x2[e] *= scale;
    }
    store_rotated_chunks<CH>(lds_row + 2 * cp * CH * 2, lds_row + (2 * cp + 1) * CH * 2, x1, x2);
}

}  // namespace attn
}  // namespace skiparse
