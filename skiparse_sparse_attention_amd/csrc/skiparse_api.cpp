// Host side of the C ABI declared in include/skiparse.h: argument validation
// (no device call before it passes), launch configuration, status codes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "../../include/skiparse.h"
#include "skiparse_index.hpp"
#include "skiparse_launch.hpp"

namespace {

using skiparse::kGroup;
using skiparse::kSingle;

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

struct Dims {
    int64_t N = 0, L = 0, elems = 0, bytes = 0;
    int esize = 0;
};

// Checks shared by every device entry point.  Fills `d` on success.  `table`: the call runs a
// kernel that keeps the whole 3D-RoPE table (one LDS row per axis position) in LDS, which bounds
// T + H + W; the kernels that evaluate a token's RoPE pairs themselves, or apply none, take any
// grid.
int check_dims(int B, int T, int H, int W, int heads, int head_dim, int sparse_k,
               int mode, int dtype, Dims* d, bool table = true) {
    if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || head_dim < 1 || sparse_k < 1)
        return SKIPARSE_E_SHAPE;
    if (mode != SKIPARSE_SINGLE && mode != SKIPARSE_GROUP) return SKIPARSE_E_UNSUPPORTED;
    if (dtype != SKIPARSE_BF16 && dtype != SKIPARSE_FP32) return SKIPARSE_E_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return SKIPARSE_E_UNSUPPORTED;
    if ((int64_t)T * H > kI32Max) return SKIPARSE_E_SHAPE;  // keeps T*H*W inside int64
    const int64_t N = (int64_t)T * H * W;
    if (N > kI32Max) return SKIPARSE_E_SHAPE;
    // every kernel indexes destination rows and (row, head, chunk) tasks in 32 bits
    const int64_t rows = (int64_t)B * N;
    if (rows > kI32Max || rows * heads > kI32Max / 8) return SKIPARSE_E_SHAPE;
    if (mode == SKIPARSE_SINGLE) {
        if (N % sparse_k) return SKIPARSE_E_DIVISIBILITY;
    } else {
        const int64_t k2 = (int64_t)sparse_k * sparse_k;
        if (k2 > N || N % k2) return SKIPARSE_E_DIVISIBILITY;
    }
    if (table && (int64_t)T + H + W > SKIPARSE_MAX_GRID_SUM) return SKIPARSE_E_UNSUPPORTED;
    d->N = N;
    d->L = N / sparse_k;
    d->esize = dtype == SKIPARSE_BF16 ? 2 : 4;
    d->elems = rows * heads * head_dim;
    d->bytes = d->elems * d->esize;
    return SKIPARSE_OK;
}

bool overlaps(const void* a, const void* b, int64_t bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

// [a, a + a_bytes) and [b, b + b_bytes) share a byte
bool ranges_overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)b_bytes && y < x + (uintptr_t)a_bytes;
}

int to_status(hipError_t e) { return e == hipSuccess ? SKIPARSE_OK : SKIPARSE_E_DEVICE; }

int remap_grid(int64_t rows) {
    // one wavefront per token row at a time, 4 per block; grid-stride loop over at most 16
    // blocks per CU of a 256-CU part (more than are resident, which keeps the memory system
    // fed while blocks start and drain)
    const int64_t blocks = (rows + 3) / 4;
    return (int)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

}  // namespace

extern "C" {

namespace {

// skiparse_validate's checks; `table` as for check_dims
int validate_attn(const void* q, const void* k, const void* v, int B, int T, int H, int W, int heads,
                  int head_dim, int sparse_k, int mode, int dtype, const void* out, bool table) {
    if (!q || !k || !v || !out) return SKIPARSE_E_NULL;
    Dims d;
    const int st = check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, table);
    if (st != SKIPARSE_OK) return st;
    // The attention kernel addresses one batch's (N, heads, head_dim) slab with 32-bit
    // offsets token*row_bytes; tokens of rows past the end of a scope (up to one
    // workgroup of queries beyond L) reach N + 256*k + k^2.
    const int64_t row_bytes = (int64_t)heads * head_dim * d.esize;
    if ((d.N + 256 * (int64_t)sparse_k + (int64_t)sparse_k * sparse_k) * row_bytes + 4096 > kI32Max)
        return SKIPARSE_E_UNSUPPORTED;
    if (overlaps(out, q, d.bytes) || overlaps(out, k, d.bytes) || overlaps(out, v, d.bytes))
        return SKIPARSE_E_ALIAS;
    return SKIPARSE_OK;
}

}  // namespace

int skiparse_validate(const void* q, const void* k, const void* v, int B, int T, int H, int W,
                      int heads, int head_dim, int sparse_k, int mode, int dtype, const void* out) {
    return validate_attn(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, true);
}

namespace {

// The forward launch shared by skiparse_attn and skiparse_attn_lse (lse may be NULL).
int attn_forward(const void* q, const void* k, const void* v, int B, int T, int H, int W, int heads,
                 int head_dim, int sparse_k, int mode, int dtype, void* out, float* lse, void* stream) {
    Dims d;
    check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d);
    skiparse::AttnParams a;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads;
    a.sparse_k = sparse_k; a.mode = mode;
    a.N = (int)d.N; a.L = (int)d.L;
    const int bm = skiparse::attn_block_rows(), bn = skiparse::attn_tile_keys();
    a.q_tiles = (int)((d.L + bm - 1) / bm);
    const int64_t work = (int64_t)B * heads * sparse_k * a.q_tiles;
    if (work > kI32Max) return SKIPARSE_E_SHAPE;
    a.num_work = (int)work;
    a.k_divides_bn = (bn % sparse_k) == 0;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    a.lse = lse;
    // consecutive rows of a scope step w by k (Single Skip) or by 1 (Group Skip)
    const int phi_div = mode == SKIPARSE_SINGLE ? sparse_k : 1;
    a.phi_mul = phi_div > 65536 ? 0 : (65536 + phi_div - 1) / phi_div;
    return to_status(skiparse::launch_attn(a, head_dim, dtype, static_cast<hipStream_t>(stream)));
}

int phi_mul_of(int mode, int sparse_k) {
    const int phi_div = mode == SKIPARSE_SINGLE ? sparse_k : 1;
    return phi_div > 65536 ? 0 : (65536 + phi_div - 1) / phi_div;
}

}  // namespace

int skiparse_attn(const void* q, const void* k, const void* v, int B, int T, int H, int W,
                  int heads, int head_dim, int sparse_k, int mode, int dtype, void* out,
                  void* stream) {
    const int st = skiparse_validate(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out);
    if (st != SKIPARSE_OK) return st;
    return attn_forward(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, nullptr, stream);
}

int skiparse_rope_qk(const void* q, const void* k, int B, int T, int H, int W, int heads, int head_dim,
                     int dtype, void* qr, void* kr, void* stream) {
    if (!q || !k || !qr || !kr) return SKIPARSE_E_NULL;
    Dims d;
    const int st = check_dims(B, T, H, W, heads, head_dim, 1, SKIPARSE_SINGLE, dtype, &d, false);
    if (st != SKIPARSE_OK) return st;
    if (head_dim != 128 || dtype != SKIPARSE_BF16) return SKIPARSE_E_UNSUPPORTED;
    if (overlaps(qr, q, d.bytes) || overlaps(qr, k, d.bytes) || overlaps(kr, q, d.bytes) ||
        overlaps(kr, k, d.bytes) || overlaps(qr, kr, d.bytes))
        return SKIPARSE_E_ALIAS;
    skiparse::RopeQkParams a;
    a.q = q; a.k = k; a.qr = qr; a.kr = kr;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.N = (int)d.N;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    return to_status(skiparse::launch_rope_qk(a, static_cast<hipStream_t>(stream)));
}

// skiparse_attn_rotated and skiparse_attn_rotated_lse (lse may be NULL)
static int attn_rotated_impl(const void* qr, const void* kr, const void* v, int B, int T, int H, int W,
                             int heads, int head_dim, int sparse_k, int mode, int dtype, void* out,
                             float* lse, void* stream) {
    const int st = validate_attn(qr, kr, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, false);
    if (st != SKIPARSE_OK) return st;
    if (head_dim != 128 || dtype != SKIPARSE_BF16 || skiparse::attn_tile_keys() % sparse_k != 0)
        return SKIPARSE_E_UNSUPPORTED;
    Dims d;
    check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, false);
    if (lse) {
        const int64_t lse_bytes = (int64_t)B * heads * d.N * 4;
        if (ranges_overlap(lse, lse_bytes, qr, d.bytes) || ranges_overlap(lse, lse_bytes, kr, d.bytes) ||
            ranges_overlap(lse, lse_bytes, v, d.bytes) || ranges_overlap(lse, lse_bytes, out, d.bytes))
            return SKIPARSE_E_ALIAS;
    }
    skiparse::AttnParams a;
    a.q = qr; a.k = kr; a.v = v; a.out = out;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads;
    a.sparse_k = sparse_k; a.mode = mode;
    a.N = (int)d.N; a.L = (int)d.L;
    const int bm = skiparse::attn_block_rows();
    a.q_tiles = (int)((d.L + bm - 1) / bm);
    const int64_t work = (int64_t)B * heads * sparse_k * a.q_tiles;
    if (work > kI32Max) return SKIPARSE_E_SHAPE;
    a.num_work = (int)work;
    a.k_divides_bn = 1;
    a.scale_log2 = 0.f;   // already folded into qr
    a.phi_mul = 0;
    a.lse = lse;
    return to_status(skiparse::launch_attn_rot(a, static_cast<hipStream_t>(stream)));
}

int skiparse_attn_rotated(const void* qr, const void* kr, const void* v, int B, int T, int H, int W,
                          int heads, int head_dim, int sparse_k, int mode, int dtype, void* out,
                          void* stream) {
    return attn_rotated_impl(qr, kr, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, nullptr, stream);
}

int skiparse_attn_rotated_lse(const void* qr, const void* kr, const void* v, int B, int T, int H, int W,
                              int heads, int head_dim, int sparse_k, int mode, int dtype, void* out,
                              float* lse, void* stream) {
    if (!lse) return SKIPARSE_E_NULL;
    return attn_rotated_impl(qr, kr, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, lse, stream);
}

int skiparse_attn_schedule(const skiparse_layer* layers, int n_layers, int B, int T, int H, int W, int heads,
                           int head_dim, int dtype, void* stream) {
    if (!layers) return SKIPARSE_E_NULL;
    if (n_layers < 1 || n_layers > 4096) return SKIPARSE_E_SHAPE;
    for (int i = 0; i < n_layers; ++i) {
        const skiparse_layer& l = layers[i];
        const int st = skiparse_validate(l.q, l.k, l.v, B, T, H, W, heads, head_dim, l.sparse_k, l.mode, dtype, l.out);
        if (st != SKIPARSE_OK) return st;
    }
    for (int i = 0; i < n_layers; ++i) {
        const skiparse_layer& l = layers[i];
        const int st = attn_forward(l.q, l.k, l.v, B, T, H, W, heads, head_dim, l.sparse_k, l.mode, dtype, l.out,
                                    nullptr, stream);
        if (st != SKIPARSE_OK) return st;
    }
    return SKIPARSE_OK;
}

int skiparse_attn_schedule_rotated(const skiparse_layer* layers, int n_layers, int B, int T, int H, int W,
                                   int heads, int head_dim, int dtype, void* qr, void* kr, void* stream) {
    if (!layers || !qr || !kr) return SKIPARSE_E_NULL;
    if (n_layers < 1 || n_layers > 4096) return SKIPARSE_E_SHAPE;
    for (int i = 0; i < n_layers; ++i) {
        const skiparse_layer& l = layers[i];
        const int st = validate_attn(l.q, l.k, l.v, B, T, H, W, heads, head_dim, l.sparse_k, l.mode, dtype, l.out,
                                     false);
        if (st != SKIPARSE_OK) return st;
        if (head_dim != 128 || dtype != SKIPARSE_BF16 || skiparse::attn_tile_keys() % l.sparse_k != 0)
            return SKIPARSE_E_UNSUPPORTED;
    }
    Dims d;
    check_dims(B, T, H, W, heads, head_dim, 1, SKIPARSE_SINGLE, dtype, &d, false);
    // the scratch rows are rewritten by every layer: they may not overlap each other or any
    // layer's buffers
    if (overlaps(qr, kr, d.bytes)) return SKIPARSE_E_ALIAS;
    for (int i = 0; i < n_layers; ++i) {
        const skiparse_layer& l = layers[i];
        const void* bufs[4] = {l.q, l.k, l.v, l.out};
        for (int j = 0; j < 4; ++j)
            if (overlaps(qr, bufs[j], d.bytes) || overlaps(kr, bufs[j], d.bytes)) return SKIPARSE_E_ALIAS;
    }
    for (int i = 0; i < n_layers; ++i) {
        const skiparse_layer& l = layers[i];
        int st = skiparse_rope_qk(l.q, l.k, B, T, H, W, heads, head_dim, dtype, qr, kr, stream);
        if (st != SKIPARSE_OK) return st;
        st = attn_rotated_impl(qr, kr, l.v, B, T, H, W, heads, head_dim, l.sparse_k, l.mode, dtype, l.out, nullptr,
                               stream);
        if (st != SKIPARSE_OK) return st;
    }
    return SKIPARSE_OK;
}

int skiparse_attn_lse(const void* q, const void* k, const void* v, int B, int T, int H, int W,
                      int heads, int head_dim, int sparse_k, int mode, int dtype, void* out,
                      float* lse, void* stream) {
    if (!lse) return SKIPARSE_E_NULL;
    const int st = skiparse_validate(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out);
    if (st != SKIPARSE_OK) return st;
    Dims d;
    check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d);
    const int64_t lse_bytes = (int64_t)B * heads * d.N * 4;
    if (ranges_overlap(lse, lse_bytes, q, d.bytes) || ranges_overlap(lse, lse_bytes, k, d.bytes) ||
        ranges_overlap(lse, lse_bytes, v, d.bytes) || ranges_overlap(lse, lse_bytes, out, d.bytes))
        return SKIPARSE_E_ALIAS;
    return attn_forward(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out, lse, stream);
}

// skiparse_attn_bwd, skiparse_attn_bwd_rotated (q, k already rotated, q scaled) and
// skiparse_attn_bwd_rotated_static (delta == nullptr: the library's static workspace)
static int attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, int B, int T, int H, int W, int heads, int head_dim,
                         int sparse_k, int mode, int dtype, void* dq, void* dk, void* dv, float* delta,
                         bool rotated, bool static_delta, void* stream) {
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || (!delta && !static_delta))
        return SKIPARSE_E_NULL;
    const int st = skiparse_validate(q, k, v, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, out);
    if (st != SKIPARSE_OK) return st;
    if (rotated && (head_dim != 128 || dtype != SKIPARSE_BF16)) return SKIPARSE_E_UNSUPPORTED;
    Dims d;
    check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d);
    const int64_t vec_bytes = (int64_t)B * heads * d.N * 4;
    // outputs: dq, dk, dv (tensor-sized) and delta (vector-sized) must not overlap any input or
    // each other (the static workspace is a buffer of its own)
    const void* ins[5] = {q, k, v, out, dout};
    void* outs[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], ins[j], d.bytes)) return SKIPARSE_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], outs[j], d.bytes)) return SKIPARSE_E_ALIAS;
        if (ranges_overlap(outs[i], d.bytes, lse, vec_bytes)) return SKIPARSE_E_ALIAS;
        if (!static_delta && ranges_overlap(outs[i], d.bytes, delta, vec_bytes)) return SKIPARSE_E_ALIAS;
    }
    if (!static_delta) {
        for (int j = 0; j < 5; ++j)
            if (ranges_overlap(delta, vec_bytes, ins[j], d.bytes)) return SKIPARSE_E_ALIAS;
        if (overlaps(delta, lse, vec_bytes)) return SKIPARSE_E_ALIAS;
    }
    skiparse::AttnBwdParams a;
    a.q = q; a.k = k; a.v = v; a.o = out; a.dout = dout; a.lse = lse; a.delta = delta;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.sparse_k = sparse_k; a.mode = mode;
    a.N = (int)d.N; a.L = (int)d.L;
    const int rows = skiparse::attn_bwd_block_rows();
    a.tiles = (int)((d.L + rows - 1) / rows);
    const int64_t work = (int64_t)B * heads * sparse_k * a.tiles;
    if (work > kI32Max) return SKIPARSE_E_SHAPE;
    a.num_work = (int)work;
    const int dq_rows = skiparse::attn_bwd_dq_rows();
    a.dq_tiles = (int)((d.L + dq_rows - 1) / dq_rows);
    a.dq_num_work = (int)((int64_t)B * heads * sparse_k * a.dq_tiles);
    a.scale = (float)(1.0 / std::sqrt((double)head_dim));
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    a.phi_mul = phi_mul_of(mode, sparse_k);
    if (static_delta) {
        if ((int64_t)B * heads * d.N > skiparse::kStaticDeltaFloats) return SKIPARSE_E_WORKSPACE;
        if (to_status(skiparse::static_delta_workspace(&a.delta)) != SKIPARSE_OK) return SKIPARSE_E_DEVICE;
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    return to_status(rotated ? skiparse::launch_attn_bwd_rot(a, hs) : skiparse::launch_attn_bwd(a, head_dim, dtype, hs));
}

int skiparse_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, int B, int T, int H, int W, int heads, int head_dim,
                      int sparse_k, int mode, int dtype, void* dq, void* dk, void* dv, float* delta,
                      void* stream) {
    return attn_backward(q, k, v, out, dout, lse, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, dq, dk, dv,
                         delta, false, false, stream);
}

int skiparse_attn_bwd_rotated(const void* qr, const void* kr, const void* v, const void* out, const void* dout,
                              const float* lse, int B, int T, int H, int W, int heads, int head_dim,
                              int sparse_k, int mode, int dtype, void* dq, void* dk, void* dv, float* delta,
                              void* stream) {
    return attn_backward(qr, kr, v, out, dout, lse, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, dq, dk, dv,
                         delta, true, false, stream);
}

int skiparse_attn_bwd_rotated_static(const void* qr, const void* kr, const void* v, const void* out,
                                     const void* dout, const float* lse, int B, int T, int H, int W, int heads,
                                     int head_dim, int sparse_k, int mode, int dtype, void* dq, void* dk,
                                     void* dv, void* stream) {
    return attn_backward(qr, kr, v, out, dout, lse, B, T, H, W, heads, head_dim, sparse_k, mode, dtype, dq, dk, dv,
                         nullptr, true, true, stream);
}

double skiparse_attn_bwd_flops(int B, int T, int H, int W, int heads, int head_dim, int sparse_k) {
    const double f = skiparse_attn_flops(B, T, H, W, heads, head_dim, sparse_k);
    return f < 0 ? f : 2.0 * f;
}

int skiparse_q8_scope_pitch(int T, int H, int W, int sparse_k) {
    if (T < 1 || H < 1 || W < 1 || sparse_k < 1) return -SKIPARSE_E_SHAPE;
    const int64_t N = (int64_t)T * H * W;
    if (N > kI32Max || N % sparse_k) return -SKIPARSE_E_DIVISIBILITY;
    return skiparse::q8_scope_pitch((int)(N / sparse_k));
}

namespace {

// Checks shared by the 8-bit calls: the attention's size limits, head_dim 128, sparse_k | 64.
int check_q8(int B, int T, int H, int W, int heads, int head_dim, int sparse_k, int mode, int dtype,
             Dims* d, int64_t* lp, bool table) {
    const int st = check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, d, table);
    if (st != SKIPARSE_OK) return st;
    if (head_dim != 128 || 64 % sparse_k != 0) return SKIPARSE_E_UNSUPPORTED;
    if ((int64_t)B * heads > 65535) return SKIPARSE_E_UNSUPPORTED;   // grid y of the statistics pass
    const int64_t row_bytes = (int64_t)heads * head_dim * d->esize;
    if ((d->N + 256 * (int64_t)sparse_k + (int64_t)sparse_k * sparse_k) * row_bytes + 4096 > kI32Max)
        return SKIPARSE_E_UNSUPPORTED;
    *lp = skiparse::q8_scope_pitch((int)d->L);
    if ((int64_t)head_dim * *lp > kI32Max) return SKIPARSE_E_UNSUPPORTED;
    return SKIPARSE_OK;
}

}  // namespace

int skiparse_quant8(const void* q, const void* k, const void* v, int B, int T, int H, int W, int heads,
                    int head_dim, int sparse_k, int mode, int dtype, void* q8, float* q_amax, void* k8,
                    float* k_amax, void* vt8, float* v_amax, void* stream) {
    if (!q || !k || !v || !q8 || !q_amax || !k8 || !k_amax || !vt8 || !v_amax) return SKIPARSE_E_NULL;
    Dims d;
    int64_t lp = 0;
    const int st = check_q8(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, &lp, true);
    if (st != SKIPARSE_OK) return st;
    const int64_t codes = (int64_t)B * d.N * heads * head_dim;
    const int64_t sizes[6] = {codes, (int64_t)B * d.N * heads * 4, codes, (int64_t)B * heads * 4,
                              (int64_t)B * heads * sparse_k * head_dim * lp, (int64_t)B * heads * head_dim * 4};
    const void* outs[6] = {q8, q_amax, k8, k_amax, vt8, v_amax};
    const void* ins[3] = {q, k, v};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 3; ++j)
            if (ranges_overlap(outs[i], sizes[i], ins[j], d.bytes)) return SKIPARSE_E_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (ranges_overlap(outs[i], sizes[i], outs[j], sizes[j])) return SKIPARSE_E_ALIAS;
    }
    skiparse::Q8Params a;
    a.q = q; a.k = k; a.v = v; a.q8 = q8; a.k8 = k8; a.vt8 = vt8;
    a.q_amax = q_amax; a.k_amax = k_amax; a.v_amax = v_amax;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.sparse_k = sparse_k; a.mode = mode;
    a.N = (int)d.N; a.Lp = (int)lp;
    return to_status(skiparse::launch_quant8(a, head_dim, dtype, static_cast<hipStream_t>(stream)));
}

int skiparse_attn8(const void* q8, const float* q_amax, const void* k8, const float* k_amax, const void* vt8,
                   const float* v_amax, int B, int T, int H, int W, int heads, int head_dim, int sparse_k,
                   int mode, int out_dtype, void* out, void* stream) {
    if (!q8 || !q_amax || !k8 || !k_amax || !vt8 || !v_amax || !out) return SKIPARSE_E_NULL;
    Dims d;
    int64_t lp = 0;
    const int st = check_q8(B, T, H, W, heads, head_dim, sparse_k, mode, out_dtype, &d, &lp, false);
    if (st != SKIPARSE_OK) return st;
    const int64_t codes = (int64_t)B * d.N * heads * head_dim;
    const int64_t sizes[6] = {codes, (int64_t)B * d.N * heads * 4, codes, (int64_t)B * heads * 4,
                              (int64_t)B * heads * sparse_k * head_dim * lp, (int64_t)B * heads * head_dim * 4};
    const void* ins[6] = {q8, q_amax, k8, k_amax, vt8, v_amax};
    for (int j = 0; j < 6; ++j)
        if (ranges_overlap(out, d.bytes, ins[j], sizes[j])) return SKIPARSE_E_ALIAS;
    skiparse::Attn8Params a;
    a.q8 = q8; a.k8 = k8; a.vt8 = vt8; a.q_amax = q_amax; a.k_amax = k_amax; a.v_amax = v_amax; a.out = out;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.sparse_k = sparse_k; a.mode = mode;
    a.N = (int)d.N; a.L = (int)d.L; a.Lp = (int)lp;
    const int rows = skiparse::attn8_block_rows();
    a.q_tiles = (int)((d.L + rows - 1) / rows);
    const int64_t work = (int64_t)B * heads * sparse_k * a.q_tiles;
    if (work > kI32Max) return SKIPARSE_E_SHAPE;
    a.num_work = (int)work;
    a.out_bytes = d.esize;
    return to_status(skiparse::launch_attn8(a, static_cast<hipStream_t>(stream)));
}

int skiparse_rope_remap(const void* q, const void* k, const void* v, int B, int T, int H, int W,
                        int heads, int head_dim, int sparse_k, int mode, int dtype, void* rq,
                        void* rk, void* rv, void* stream) {
    if (!q || !k || !v || !rq || !rk || !rv) return SKIPARSE_E_NULL;
    Dims d;
    const bool pairs_per_row = head_dim == 128 && dtype == SKIPARSE_BF16;
    const int st = check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, !pairs_per_row);
    if (st != SKIPARSE_OK) return st;
    const void* ins[3] = {q, k, v};
    void* outs[3] = {rq, rk, rv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlaps(outs[i], ins[j], d.bytes)) return SKIPARSE_E_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], outs[j], d.bytes)) return SKIPARSE_E_ALIAS;
    }
    skiparse::RemapParams a;
    for (int i = 0; i < 3; ++i) { a.src[i] = ins[i]; a.dst[i] = outs[i]; }
    a.ntensors = 3;
    a.rope_mask = 0x3;  // q and k are rotated, v is moved unchanged
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.k = sparse_k; a.mode = mode;
    a.L = (int)d.L; a.N = (int)d.N; a.rows = (int)(B * d.N);
    return to_status(skiparse::launch_rope_remap(a, head_dim, dtype, static_cast<hipStream_t>(stream),
                                                 remap_grid(a.rows)));
}

int skiparse_rearrange(const void* x, int B, int T, int H, int W, int heads, int head_dim,
                       int sparse_k, int mode, int dtype, int apply_rope, void* out, void* stream) {
    if (!x || !out) return SKIPARSE_E_NULL;
    Dims d;
    const bool pairs_per_row = head_dim == 128 && dtype == SKIPARSE_BF16;
    const int st = check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, apply_rope && !pairs_per_row);
    if (st != SKIPARSE_OK) return st;
    if (overlaps(out, x, d.bytes)) return SKIPARSE_E_ALIAS;
    skiparse::RemapParams a;
    a.src[0] = x; a.dst[0] = out;
    a.src[1] = a.src[2] = nullptr;
    a.dst[1] = a.dst[2] = nullptr;
    a.ntensors = 1;
    a.rope_mask = apply_rope ? 1 : 0;
    a.B = B; a.T = T; a.H = H; a.W = W; a.heads = heads; a.k = sparse_k; a.mode = mode;
    a.L = (int)d.L; a.N = (int)d.N; a.rows = (int)(B * d.N);
    return to_status(skiparse::launch_rope_remap(a, head_dim, dtype, static_cast<hipStream_t>(stream),
                                                 remap_grid(a.rows)));
}

int skiparse_reverse(const void* x, int B, int T, int H, int W, int heads, int head_dim,
                     int sparse_k, int mode, int dtype, void* out, void* stream) {
    if (!x || !out) return SKIPARSE_E_NULL;
    Dims d;
    const int st = check_dims(B, T, H, W, heads, head_dim, sparse_k, mode, dtype, &d, false);
    if (st != SKIPARSE_OK) return st;
    if (overlaps(out, x, d.bytes)) return SKIPARSE_E_ALIAS;
    skiparse::ReverseParams a;
    a.src = x; a.dst = out;
    a.B = B; a.N = (int)d.N; a.k = sparse_k; a.mode = mode; a.L = (int)d.L;
    a.rows = (int)(B * d.N);
    a.row_bytes = (uint32_t)(heads * head_dim * d.esize);
    return to_status(skiparse::launch_reverse(a, static_cast<hipStream_t>(stream),
                                              remap_grid(a.rows)));
}

int skiparse_scope_table(int64_t N, int sparse_k, int mode, int64_t* token_of) {
    if (!token_of) return SKIPARSE_E_NULL;
    if (N < 1 || sparse_k < 1) return SKIPARSE_E_SHAPE;
    if (mode != SKIPARSE_SINGLE && mode != SKIPARSE_GROUP) return SKIPARSE_E_UNSUPPORTED;
    const int64_t k = sparse_k;
    if (mode == SKIPARSE_SINGLE ? (N % k) : (k * k > N || N % (k * k))) return SKIPARSE_E_DIVISIBILITY;
    const int64_t L = N / k;
    for (int64_t s = 0; s < k; ++s)
        for (int64_t p = 0; p < L; ++p) token_of[s * L + p] = skiparse::scope_token(p, s, k, mode);
    return SKIPARSE_OK;
}

double skiparse_attn_flops(int B, int T, int H, int W, int heads, int head_dim, int sparse_k) {
    if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || head_dim < 1 || sparse_k < 1) return -1.0;
    const double N = (double)T * H * W;
    return 4.0 * B * heads * N * std::floor(N / sparse_k) * head_dim;
}

int skiparse_probe_mfma(int blocks, int iters, float* out, void* stream) {
    if (!out) return SKIPARSE_E_NULL;
    if (blocks < 1 || iters < 1 || blocks > (1 << 20)) return SKIPARSE_E_SHAPE;
    return to_status(skiparse::launch_probe_mfma(blocks, iters, out, static_cast<hipStream_t>(stream)));
}

double skiparse_probe_mfma_flops(int blocks, int iters) {
    if (blocks < 1 || iters < 1) return -1.0;
    // waves per block x products per wave (four chains) x 2*32*32*16 FLOP
    return (double)blocks * (skiparse::probe_threads() / 64) * 4.0 * iters * (2.0 * 32 * 32 * 16);
}

int skiparse_probe_stream(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
    if (!src || !dst) return SKIPARSE_E_NULL;
    if (bytes < 16 || bytes % 16 || blocks < 1 || blocks > (1 << 20)) return SKIPARSE_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return SKIPARSE_E_UNSUPPORTED;
    if (overlaps(src, dst, bytes)) return SKIPARSE_E_ALIAS;
    return to_status(skiparse::launch_probe_stream(src, dst, bytes / 16, blocks, static_cast<hipStream_t>(stream)));
}

const char* skiparse_status_string(int status) {
    switch (status) {
        case SKIPARSE_OK: return "ok";
        case SKIPARSE_E_NULL: return "a required pointer is NULL";
        case SKIPARSE_E_SHAPE: return "a size is < 1 or a size product overflows";
        case SKIPARSE_E_DIVISIBILITY: return "N is not divisible by k (Single Skip) or k^2 (Group Skip)";
        case SKIPARSE_E_UNSUPPORTED: return "unsupported head_dim, mode, dtype or grid size";
        case SKIPARSE_E_ALIAS: return "an output buffer overlaps an input buffer";
        case SKIPARSE_E_DEVICE: return "a HIP call failed";
        case SKIPARSE_E_WORKSPACE: return "B*heads*N exceeds the static workspace";
        default: return "unknown status";
    }
}

const char* skiparse_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
