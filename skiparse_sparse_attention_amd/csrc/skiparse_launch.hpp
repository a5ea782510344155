// Kernel parameter blocks and launchers (internal to the library; the public
// interface is include/skiparse.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/skiparse.h"

namespace skiparse {

constexpr int kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit, the most one workgroup can take

struct RemapParams {
    const void* src[3];
    void* dst[3];
    int ntensors;   // 1 or 3
    int rope_mask;  // bit i set: rotate tensor i by 3D RoPE before moving it
    int B, T, H, W, heads, k, mode, L, N;
    int rows;       // B*N destination rows
};

struct ReverseParams {
    const void* src;
    void* dst;
    int B, N, k, mode, L;
    int rows;          // B*N
    uint32_t row_bytes;  // heads*head_dim*element size (multiple of 16)
};

struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, T, H, W, heads, sparse_k, mode, N, L;
    int q_tiles;     // ceil(L / BM)
    int num_work;    // B*heads*sparse_k*q_tiles workgroups
    int k_divides_bn;  // sparse_k divides the key-tile height
    float scale_log2;  // log2(e) / sqrt(head_dim)
    int phi_mul;       // ceil(2^16 / phi_div), phi_div = w step between consecutive scope rows
    float* lse;        // optional (B, heads, N) fp32: log2 of each row's softmax denominator,
                       // in the units of the scores scaled by scale_log2
};

struct AttnBwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;       // forward output
    const void* dout;    // gradient of the loss with respect to the output
    const float* lse;    // (B, heads, N): the forward's log2-sum-exp of each row
    float* delta;        // (B, heads, N) workspace: rowsum(dout * o), written by the dq kernel
    void* dq;
    void* dk;
    void* dv;
    int B, T, H, W, heads, sparse_k, mode, N, L;
    int tiles;           // ceil(L / 128): key tiles of the dk/dv kernel
    int num_work;        // B*heads*sparse_k*tiles workgroups of the dk/dv kernel
    int dq_tiles;        // ceil(L / 256): query tiles of the dq kernel
    int dq_num_work;     // B*heads*sparse_k*dq_tiles workgroups of the dq kernel
    float scale_log2;    // log2(e) / sqrt(head_dim)
    float scale;         // 1 / sqrt(head_dim)
    int phi_mul;
};

// 8-bit operands (quant8.hip): q8, k8 int8 (B, N, heads, d); vt8 E4M3 (B, heads, k, d, Lp)
struct Q8Params {
    const void* q;
    const void* k;
    const void* v;
    void* q8;
    void* k8;
    void* vt8;
    float* q_amax;       // (B, N, heads)
    float* k_amax;       // (B, heads)
    float* v_amax;       // (B, heads, d)
    int B, T, H, W, heads, sparse_k, mode, N;
    int Lp;              // L rounded up to a multiple of 64: the channel-row pitch of vt8
};

// 8-bit attention (attn8_fwd.hip), operands from quant8.hip
struct Attn8Params {
    const void* q8;
    const void* k8;
    const void* vt8;
    const float* q_amax;
    const float* k_amax;
    const float* v_amax;
    void* out;
    int B, T, H, W, heads, sparse_k, mode, N, L, Lp;
    int q_tiles;         // ceil(L / 256)
    int num_work;        // B*heads*sparse_k*q_tiles workgroups
    int out_bytes;       // 2 (bf16) or 4 (fp32)
};

// Pre-rotated operands (attn_rot.hip): qr = bf16(RoPE(q) * scale_log2), kr = bf16(RoPE(k)),
// both (B, N, heads, 128) in token order; the attention on them takes AttnParams with q = qr,
// k = kr (bf16 only, sparse_k dividing 64).
struct RopeQkParams {
    const void* q;
    const void* k;
    void* qr;
    void* kr;
    int B, T, H, W, heads, N;
    float scale_log2;
};

hipError_t launch_rope_remap(const RemapParams& a, int head_dim, int dtype, hipStream_t stream, int grid);
hipError_t launch_reverse(const ReverseParams& a, hipStream_t stream, int grid);
hipError_t launch_attn(const AttnParams& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_attn_bwd(const AttnBwdParams& a, int head_dim, int dtype, hipStream_t stream);
int attn_block_rows();  // query rows per attention workgroup
int attn_bwd_block_rows();  // keys per dk/dv workgroup
int attn_bwd_dq_rows();     // queries per dq workgroup
int attn_tile_keys();   // keys per attention K/V tile
hipError_t launch_quant8(const Q8Params& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_attn8(const Attn8Params& a, hipStream_t stream);
int q8_scope_pitch(int L);  // Lp of the vt8 layout
int attn8_block_rows();     // query rows per 8-bit attention workgroup
hipError_t launch_rope_qk(const RopeQkParams& a, hipStream_t stream);
hipError_t launch_attn_rot(const AttnParams& a, hipStream_t stream);   // a.lse set: also writes it
hipError_t launch_attn_bwd_rot(const AttnBwdParams& a, hipStream_t stream);
// Capacity (fp32 elements) of the static delta workspace and its address on the current device.
constexpr int64_t kStaticDeltaFloats = SKIPARSE_STATIC_DELTA_MAX;   // 16 MiB per GPU
hipError_t static_delta_workspace(float** ptr);
// measurement probes
hipError_t launch_probe_mfma(int blocks, int iters, float* out, hipStream_t stream);
hipError_t launch_probe_stream(const void* src, void* dst, int64_t pieces, int blocks, hipStream_t stream);
int probe_threads();

}  // namespace skiparse
