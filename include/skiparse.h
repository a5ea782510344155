/*
 * skiparse.h -- C ABI of the MI355X (gfx950) Skiparse attention library.
 *
 * Skiparse attention (Open-Sora Plan documentation, section "Skiparse
 * Attention") splits the token sequence of a full-3D-attention block into
 * sparse_k scopes and runs softmax attention inside each scope only:
 *
 *   1. 3D RoPE on q and k, at each token's original (t, h, w) grid position
 *      (the page's implementation note: RoPE goes before the rearrange);
 *   2. the Single Skip or Group Skip rearrange of q, k, v into sparse_k scopes
 *      of L = N / sparse_k tokens (the page's einops patterns);
 *   3. softmax(Q K^T / sqrt(head_dim)) V inside each scope, per head
 *      (the page's scaled_dot_product_attention call: no mask, non-causal);
 *   4. the inverse rearrange back to the original token order.
 *
 * With sparse_k == 1 this is dense full-3D attention.
 *
 * Two forms of the same computation, with bit-identical results:
 *   - skiparse_attn (+ _lse, _bwd): one launch, RoPE applied inside the
 *     attention kernel's tile loads;
 *   - skiparse_rope_qk, then skiparse_attn_rotated (+ _lse, skiparse_attn_bwd_rotated):
 *     step 1 as its own pass, whose output serves any number of attentions
 *     over the same q and k; head_dim 128, bf16.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Token layout.  q, k, v and out are dense, contiguous (B, N, heads, head_dim)
 *   arrays, N = T*H*W, token n = (t*H + h)*W + w (Wan 2.1 report, section
 *   4.2.1: the patchified latent is flattened frame-major into a (B, L, D)
 *   sequence).  This is the page's (B, N, C) layout with C = heads*head_dim.
 * Scopes.  Single Skip (mode 0): token n is in scope s = n mod k at in-scope
 *   position p = n div k.  Group Skip (mode 1): token n is in scope
 *   s = (n div k) mod k at position p = (n div k^2)*k + n mod k.  In-scope order
 *   is increasing token index; a rearranged tensor puts the scope axis in front
 *   of the batch axis (row s*B + b), the layout of the page's Single Skip and
 *   Group Skip code.
 * 3D RoPE.  head_dim is split 2:3:3 over the t, h, w axes (16/24/24 at
 *   head_dim 64, 32/48/48 at 128), in that order.  Inside an axis chunk of size
 *   d_a, slot j and slot j + d_a/2 form a rotate-half pair rotated by
 *   pos_a * 10000^(-2j/d_a):  x1' = x1 cos - x2 sin,  x2' = x2 cos + x1 sin.
 *   The pages use RoPE without defining it; this is the reading the library
 *   implements.
 * Precision.  dtype SKIPARSE_BF16: bf16 in, bf16 out, RoPE in fp32, attention
 *   operands bf16 on the matrix cores with fp32 accumulation and fp32 softmax.
 *   dtype SKIPARSE_FP32: fp32 in and out; attention rounds its rotated fp32
 *   operands to bf16 at tile load (same arithmetic as bf16 otherwise); the
 *   rearrange/reverse calls keep fp32 throughout.
 * Pointers.  All array pointers are device pointers (hipMalloc'd or torch CUDA
 *   tensors' data_ptr), 16-byte aligned.  The caller owns every buffer; the
 *   library allocates nothing and keeps no state between calls, except the
 *   static workspace of skiparse_attn_bwd_rotated_static (one per GPU, for the
 *   life of the process).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL: the default
 *   stream).  Calls are asynchronous: they return once the kernels are
 *   enqueued; execution errors surface at the caller's next synchronization.
 * Errors.  Every call validates its arguments on the host before any device
 *   call and returns a skiparse_status; nothing aborts or prints.
 */
#ifndef SKIPARSE_H
#define SKIPARSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum skiparse_mode { SKIPARSE_SINGLE = 0, SKIPARSE_GROUP = 1 };
enum skiparse_dtype { SKIPARSE_BF16 = 0, SKIPARSE_FP32 = 1 };

enum skiparse_status {
    SKIPARSE_OK = 0,
    SKIPARSE_E_NULL = 1,          /* a required pointer is NULL                              */
    SKIPARSE_E_SHAPE = 2,         /* a size is < 1, or a size product overflows              */
    SKIPARSE_E_DIVISIBILITY = 3,  /* Single: N % k != 0; Group: N % k^2 != 0 (no padding)     */
    SKIPARSE_E_UNSUPPORTED = 4,   /* head_dim not 64/128, bad mode/dtype, grid too large     */
    SKIPARSE_E_ALIAS = 5,         /* an output buffer overlaps an input buffer               */
    SKIPARSE_E_DEVICE = 6,        /* a HIP call failed (launch error, no device, ...)        */
    SKIPARSE_E_WORKSPACE = 7      /* B*heads*N exceeds SKIPARSE_STATIC_DELTA_MAX (the static
                                     workspace of skiparse_attn_bwd_rotated_static only)    */
};

/* Largest T + H + W for the calls whose kernels keep the whole 3D-RoPE cos/sin table,
 * one row per axis position, in LDS (256 bytes per row beside each kernel's tile buffers;
 * at 224 rows the rotated dk/dv kernel, the largest, fills 163,328 of its 163,840 bytes):
 * skiparse_attn, skiparse_attn_lse, skiparse_attn_schedule, both
 * backward calls, skiparse_quant8, and skiparse_rope_remap / skiparse_rearrange with RoPE
 * at a dtype or head_dim other than bf16 / 128.  They return SKIPARSE_E_UNSUPPORTED for
 * larger grids.  skiparse_rope_qk, skiparse_attn_rotated(_lse),
 * skiparse_attn_schedule_rotated, skiparse_attn8, skiparse_reverse and the bf16 /
 * head_dim 128 remap evaluate each token's RoPE pairs themselves (or apply none) and take
 * any grid within the other size limits. */
#define SKIPARSE_MAX_GRID_SUM 224

/*
 * skiparse_attn -- the fused Skiparse attention forward (steps 1-4 above).
 *
 * q, k, v : (B, N, heads, head_dim) inputs in `dtype`, N = T*H*W.
 * out     : (B, N, heads, head_dim) output in `dtype`, in the original token
 *           order; must not overlap q, k or v.
 * sparse_k: number of scopes k >= 1 (Single: N % k == 0; Group: N % k^2 == 0).
 * head_dim: 64 or 128.
 * Limit: the kernel addresses one batch's (N, heads, head_dim) slab with
 * 32-bit byte offsets, so (N + 256*k + k^2) * heads*head_dim*sizeof(dtype)
 * + 4096 must stay below 2^31 (about 2 GiB per batch); larger inputs return
 * SKIPARSE_E_UNSUPPORTED.
 * One kernel launch.  The rearranged q, k, v are never written to memory:
 * each tile load gathers its scope's rows and rotates them on the fly, and
 * the epilogue writes each output row straight to its original token index.
 * Returns SKIPARSE_OK or an error code; the output is not touched on error.
 */
int skiparse_attn(const void* q, const void* k, const void* v,
                  int B, int T, int H, int W, int heads, int head_dim,
                  int sparse_k, int mode, int dtype, void* out, void* stream);

/*
 * skiparse_attn_lse -- skiparse_attn that also writes, for the backward pass,
 * each output row's log2-sum-exp.
 *
 * Everything as skiparse_attn, plus
 * lse : (B, heads, N) fp32, device memory, caller-owned; entry
 *       [b, head, n] = log2 of sum_m 2^(z_nm), with z_nm = (q'_n . k'_m) *
 *       log2(e) / sqrt(head_dim) over the members m of token n's scope (q', k'
 *       the rotated rows): the softmax denominator of row n in base-2 units of
 *       the scaled scores.  Must not overlap q, k, v or out.
 * The same single kernel launch; the rows of lse are written in its epilogue.
 */
int skiparse_attn_lse(const void* q, const void* k, const void* v,
                      int B, int T, int H, int W, int heads, int head_dim,
                      int sparse_k, int mode, int dtype, void* out, float* lse,
                      void* stream);

/*
 * skiparse_rope_qk -- the 3D RoPE of q and k, once, for any number of Skiparse
 * attentions over them (Open-Sora Plan documentation, "Skiparse Attention":
 * q and k are rotated at their original token positions before the scopes are
 * formed, so the rotation is the same for every k and mode).
 *
 * q, k   : (B, N, heads, 128) bf16 inputs, N = T*H*W (device memory).
 * qr, kr : (B, N, heads, 128) bf16 outputs, caller-owned, in token order:
 *          qr = bf16(RoPE(q) * log2(e)/sqrt(128)) -- the softmax scale in base-2
 *          units folded in -- and kr = bf16(RoPE(k)), each element computed as
 *          skiparse_attn computes its operands (same cos/sin table, same float32
 *          operations), so they are bit for bit the operands skiparse_attn feeds
 *          its matrix cores.  No output may overlap an input or the other output.
 * head_dim must be 128 and dtype SKIPARSE_BF16 (else SKIPARSE_E_UNSUPPORTED);
 * other limits as skiparse_attn.  One kernel launch; outputs untouched on error.
 */
int skiparse_rope_qk(const void* q, const void* k, int B, int T, int H, int W,
                     int heads, int head_dim, int dtype, void* qr, void* kr,
                     void* stream);

/*
 * skiparse_attn_rotated -- skiparse_attn on operands from skiparse_rope_qk:
 * the gather, attention and scatter of skiparse_attn (steps 2-4 above) with
 * RoPE and the softmax scale already applied.
 *
 * qr, kr : outputs of skiparse_rope_qk for the same B, grid, heads.
 * v, out : as skiparse_attn.  out must not overlap qr, kr or v.
 * head_dim 128, dtype SKIPARSE_BF16 and sparse_k dividing 64 (else
 * SKIPARSE_E_UNSUPPORTED); other limits as skiparse_attn.
 * skiparse_rope_qk followed by skiparse_attn_rotated gives out equal to
 * skiparse_attn's bit for bit.  One kernel launch; out untouched on error.
 */
int skiparse_attn_rotated(const void* qr, const void* kr, const void* v,
                          int B, int T, int H, int W, int heads, int head_dim,
                          int sparse_k, int mode, int dtype, void* out,
                          void* stream);

/*
 * skiparse_attn_rotated_lse -- skiparse_attn_rotated that also writes, for the
 * backward pass, each output row's log2-sum-exp.
 *
 * Everything as skiparse_attn_rotated, plus lse: (B, heads, N) fp32, device
 * memory, caller-owned, with the meaning given at skiparse_attn_lse; must not
 * overlap qr, kr, v or out.  out and lse equal skiparse_attn_lse's on the
 * unrotated q, k bit for bit.  One kernel launch.
 */
int skiparse_attn_rotated_lse(const void* qr, const void* kr, const void* v,
                              int B, int T, int H, int W, int heads, int head_dim,
                              int sparse_k, int mode, int dtype, void* out, float* lse,
                              void* stream);

/*
 * skiparse_attn_bwd -- gradients of a loss through skiparse_attn (the chain
 * rule of steps 1-4, taken backwards).  Open-Sora Plan's page says Skiparse
 * exists to speed up training; these are the gradients training needs.
 *
 * q, k, v : the forward inputs, (B, N, heads, head_dim) in `dtype`.
 * out     : the forward output (skiparse_attn_lse's out), same layout.
 * dout    : gradient of the loss with respect to out, same layout.
 * lse     : skiparse_attn_lse's log2-sum-exp of the same call, (B, heads, N) fp32.
 * dq, dk, dv : gradients with respect to q, k, v, (B, N, heads, head_dim) in
 *           `dtype`, original token order; dq and dk include the transposed RoPE
 *           rotation (each rotate-half pair turned back by -theta).
 * delta   : (B, heads, N) fp32 workspace, caller-owned: receives
 *           rowsum(dout * out) of every row (written, then read, by this call).
 * Per scope, with Z = q' k'^T / sqrt(d) and P = softmax(Z):
 *   dv = P^T dout,  dZ = P * (dout v^T - delta),  dq' = dZ k' / sqrt(d),
 *   dk' = dZ^T q' / sqrt(d),  dq and dk = the transposed RoPE of dq', dk'.
 * Precision: bf16 operands on the matrix cores, fp32 accumulation, P and dZ
 *   rounded to bf16 as MFMA operands, delta and the rotations in fp32.
 * Two kernel launches on `stream` (dq and delta first, then dk and dv).  No
 * output (dq, dk, dv, delta) may overlap any input or another output.  Same
 * size limits as skiparse_attn.  Returns SKIPARSE_OK or an error code.
 */
int skiparse_attn_bwd(const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse,
                      int B, int T, int H, int W, int heads, int head_dim,
                      int sparse_k, int mode, int dtype,
                      void* dq, void* dk, void* dv, float* delta, void* stream);

/*
 * skiparse_attn_bwd_rotated -- skiparse_attn_bwd with q and k given as the
 * outputs of skiparse_rope_qk (qr, kr: rotated, qr also scaled).  out and lse
 * come from skiparse_attn_rotated_lse (or skiparse_attn_lse) on the same
 * inputs.  dq and dk are still the gradients with respect to the unrotated
 * q and k (rotated back inside the kernels), dv with respect to v; they equal
 * skiparse_attn_bwd's bit for bit.  head_dim 128 and dtype SKIPARSE_BF16 only
 * (else SKIPARSE_E_UNSUPPORTED); every other rule as skiparse_attn_bwd.  Two
 * kernel launches.
 */
int skiparse_attn_bwd_rotated(const void* qr, const void* kr, const void* v,
                              const void* out, const void* dout, const float* lse,
                              int B, int T, int H, int W, int heads, int head_dim,
                              int sparse_k, int mode, int dtype,
                              void* dq, void* dk, void* dv, float* delta, void* stream);

/* Capacity of skiparse_attn_bwd_rotated_static's workspace: B*heads*N fp32
 * values (16 MiB per GPU). */
#define SKIPARSE_STATIC_DELTA_MAX 4194304

/*
 * skiparse_attn_bwd_rotated_static -- skiparse_attn_bwd_rotated without the
 * delta argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc).  The delta vector lives in a static device array of the library
 * (SKIPARSE_STATIC_DELTA_MAX fp32 values, 256-byte aligned), one per GPU,
 * held from the library's load until the process ends; its address on each
 * device is looked up once, on the first call with that device current.  The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * Everything else -- arguments, layouts, limits, results (bit for bit) -- is
 * skiparse_attn_bwd_rotated's.  B*heads*N above SKIPARSE_STATIC_DELTA_MAX
 * returns SKIPARSE_E_WORKSPACE before any device call.
 * Every call on one GPU shares that GPU's workspace: each call writes all of
 * the delta it reads (nothing needs to start at zero), but calls that overlap
 * in time on one GPU -- on different streams, or from different threads --
 * race on it and must be serialised by the caller.
 */
int skiparse_attn_bwd_rotated_static(const void* qr, const void* kr, const void* v,
                                     const void* out, const void* dout, const float* lse,
                                     int B, int T, int H, int W, int heads, int head_dim,
                                     int sparse_k, int mode, int dtype,
                                     void* dq, void* dk, void* dv, void* stream);

/*
 * skiparse_attn_bwd_flops -- FLOPs counted for one skiparse_attn_bwd call:
 * twice the forward's (Wan 2.1 report, section 4.3.1: the backward of
 * non-causal attention costs 8*b*s^2*h against 4 forward), i.e.
 * 8*B*heads*N*(N/k)*head_dim.  Negative for invalid sizes.
 */
double skiparse_attn_bwd_flops(int B, int T, int H, int W, int heads, int head_dim,
                               int sparse_k);

/*
 * 8-bit Skiparse attention (Wan 2.1 report, section 4.4.3 "Quantization",
 * paragraph "8-Bit FlashAttention": Int8 operands for S = Q K^T, FP8 (E4M3)
 * operands for O = P V, float32 accumulation across key blocks).  Two calls:
 * skiparse_quant8 turns bf16/fp32 q, k, v into the 8-bit operands, and
 * skiparse_attn8 runs the attention on them.  head_dim 128 only; sparse_k must
 * divide 64; B*heads at most 65535 (SKIPARSE_E_UNSUPPORTED otherwise).
 *
 * Operand layouts (all device memory, caller-owned, N = T*H*W, L = N/sparse_k,
 * Lp = skiparse_q8_scope_pitch(T, H, W, sparse_k) = L rounded up to 64):
 *   q8, k8 : int8 (B, N, heads, 128), original token order, codes of q' and k'
 *            (q, k after the same 3D RoPE as skiparse_attn, in float32);
 *   q_amax : float32 (B, N, heads), max |q'| over each head row;
 *   k_amax : float32 (B, heads), max |k'| over every token and channel;
 *   vt8    : uint8 E4M3 codes (B, heads, sparse_k, 128, Lp): entry
 *            [b, head, s, c, p] encodes v[b, n(s, p), head, c] * (448 / v_amax),
 *            n(s, p) the token at position p of scope s; positions p >= L hold 0;
 *   v_amax : float32 (B, heads, 128), max |v| over the tokens of each channel.
 * Codes: round-half-even(x * (127 / amax)) for int8, E4M3 round-to-nearest-even
 * for V; the reciprocal and the product are float32 operations rounded once
 * each, and a zero amax gives zero codes.
 */

/*
 * skiparse_q8_scope_pitch -- Lp, the channel-row pitch (in keys) of vt8: L
 * rounded up to a multiple of 64.  Host only; negative status for invalid
 * sizes.
 */
int skiparse_q8_scope_pitch(int T, int H, int W, int sparse_k);

/*
 * skiparse_quant8 -- the 8-bit operands of q, k, v (layouts above).
 * q, k, v : (B, N, heads, head_dim) in `dtype` (SKIPARSE_BF16 or SKIPARSE_FP32).
 * Outputs q8, q_amax, k8, k_amax, vt8, v_amax must not overlap any input or
 * each other.  Three kernel launches on `stream`: a fill of k_amax and v_amax
 * with zeros, a pass folding |k'| and |v| maxima into them with atomic maxima,
 * and the quantisation pass.  Returns SKIPARSE_OK or an error code.
 */
int skiparse_quant8(const void* q, const void* k, const void* v,
                    int B, int T, int H, int W, int heads, int head_dim,
                    int sparse_k, int mode, int dtype,
                    void* q8, float* q_amax, void* k8, float* k_amax,
                    void* vt8, float* v_amax, void* stream);

/*
 * skiparse_attn8 -- 8-bit Skiparse attention of skiparse_quant8's operands.
 * For query token i of scope s and the scope's keys j:
 *   z_ij = (q8_i . k8_j) * (q_amax_i/127) * (k_amax/127) * log2(e) / sqrt(128)
 *   M_i  = ceil(max_j z_ij),  P_ij = 2^(z_ij - M_i + 8)
 *   out_i = (sum_j E4M3(P_ij) * V~_j) * (v_amax / 448) / sum_j P_ij
 * (V~ the decoded vt8 codes), written to token i's row of out.
 * out : (B, N, heads, 128) in `out_dtype` (SKIPARSE_BF16 or SKIPARSE_FP32),
 *       must not overlap any operand.  One kernel launch.  Same size limits as
 *       skiparse_attn.  Returns SKIPARSE_OK or an error code.
 */
int skiparse_attn8(const void* q8, const float* q_amax, const void* k8,
                   const float* k_amax, const void* vt8, const float* v_amax,
                   int B, int T, int H, int W, int heads, int head_dim,
                   int sparse_k, int mode, int out_dtype, void* out, void* stream);

/*
 * A per-layer schedule of Skiparse attention calls.  Open-Sora Plan's feature
 * list describes SUV as a U-shaped sparse structure over the transformer's
 * layers without giving the per-layer sparsity; a schedule is the knob that
 * expresses one: every layer may use its own sparse_k and mode.
 */
typedef struct skiparse_layer {
    const void* q;     /* (B, N, heads, head_dim) in the schedule's dtype */
    const void* k;
    const void* v;
    void* out;         /* same layout; must not overlap this layer's q, k, v */
    int sparse_k;
    int mode;          /* SKIPARSE_SINGLE or SKIPARSE_GROUP */
} skiparse_layer;

/*
 * skiparse_attn_schedule -- run n_layers skiparse_attn calls, layers[i] with
 * its own buffers, sparse_k and mode, all on `stream` in order.  Every layer
 * is validated first (same rules as skiparse_attn); if any is invalid nothing
 * is launched and the status of the first invalid layer is returned.  Each
 * layer is one kernel launch with no host synchronisation between them; the
 * call allocates nothing and issues no memset, so a caller may capture it in a
 * HIP graph and replay the whole schedule.  Results equal those of separate
 * skiparse_attn calls bit for bit.  n_layers in [1, 4096].
 */
int skiparse_attn_schedule(const skiparse_layer* layers, int n_layers,
                           int B, int T, int H, int W, int heads, int head_dim,
                           int dtype, void* stream);

/*
 * skiparse_attn_schedule_rotated -- skiparse_attn_schedule with every layer run as
 * skiparse_rope_qk into the caller's scratch (qr, kr: (B, N, heads, 128) bf16 each,
 * rewritten by every layer; they must not overlap each other or any layer's q, k,
 * v, out) followed by skiparse_attn_rotated.  Results equal skiparse_attn_schedule's
 * bit for bit.  head_dim 128, dtype SKIPARSE_BF16 and every layer's sparse_k
 * dividing 64 (else SKIPARSE_E_UNSUPPORTED); all layers are validated before the
 * first launch; two launches per layer, no allocation or memset (capturable in a
 * HIP graph).
 */
int skiparse_attn_schedule_rotated(const skiparse_layer* layers, int n_layers,
                                   int B, int T, int H, int W, int heads, int head_dim,
                                   int dtype, void* qr, void* kr, void* stream);

/*
 * skiparse_rope_remap -- the materialised RoPE + rearrange of q, k and v in
 * one pass (the page's add_rope + *_skip_rearrange calls, before attention).
 *
 * q, k, v    : (B, N, heads, head_dim) inputs in `dtype`.
 * rq, rk, rv : (sparse_k*B, N/sparse_k, heads, head_dim) outputs in `dtype`;
 *              row s*B + b holds scope s of batch b (the page's '(k b)' /
 *              '(m b)' batch order).  rq, rk are rotated by 3D RoPE at each
 *              token's original position; rv is moved unchanged.
 * No output may overlap any input.  One kernel launch.
 */
int skiparse_rope_remap(const void* q, const void* k, const void* v,
                        int B, int T, int H, int W, int heads, int head_dim,
                        int sparse_k, int mode, int dtype,
                        void* rq, void* rk, void* rv, void* stream);

/*
 * skiparse_rearrange -- one tensor: (B, N, heads, head_dim) ->
 * (sparse_k*B, N/sparse_k, heads, head_dim), optionally rotated by 3D RoPE
 * first (apply_rope != 0).  With apply_rope == 0 the bytes are moved
 * unchanged (bit-exact for either dtype).  out must not overlap x.
 */
int skiparse_rearrange(const void* x, int B, int T, int H, int W, int heads,
                       int head_dim, int sparse_k, int mode, int dtype,
                       int apply_rope, void* out, void* stream);

/*
 * skiparse_reverse -- the page's reverse_sparse: (sparse_k*B, N/sparse_k,
 * heads, head_dim) -> (B, N, heads, head_dim), bytes moved unchanged.
 * out must not overlap x.
 */
int skiparse_reverse(const void* x, int B, int T, int H, int W, int heads,
                     int head_dim, int sparse_k, int mode, int dtype,
                     void* out, void* stream);

/*
 * skiparse_validate -- the argument checks skiparse_attn performs, with no
 * device call (host-only; usable without a GPU).  Pointers may be any
 * non-NULL values; only their ranges are compared for overlap.
 */
int skiparse_validate(const void* q, const void* k, const void* v,
                      int B, int T, int H, int W, int heads, int head_dim,
                      int sparse_k, int mode, int dtype, const void* out);

/*
 * skiparse_scope_table -- host-only: fills token_of[s*(N/k) + p] with the
 * token index at position p of scope s (int64, k*(N/k) = N entries, caller-owned).
 * The same index arithmetic the kernels use.  Returns SKIPARSE_OK, or
 * E_NULL / E_SHAPE / E_DIVISIBILITY / E_UNSUPPORTED on bad arguments.
 */
int skiparse_scope_table(int64_t N, int sparse_k, int mode, int64_t* token_of);

/*
 * skiparse_attn_flops -- FLOPs counted for one skiparse_attn call:
 * 4*B*heads*N*(N/k)*head_dim (Wan 2.1 report, section 4.3.1: non-causal
 * forward attention costs 4*b*s^2*h, here over k scopes of length N/k).
 * Returns a negative value for invalid sizes.
 */
double skiparse_attn_flops(int B, int T, int H, int W, int heads, int head_dim,
                           int sparse_k);

/*
 * Measurement probes (not part of the method).  They measure, on the part
 * itself, the two ceilings the kernels above are compared against: the
 * matrix-core rate and the streaming copy rate of HBM.
 *
 * skiparse_probe_mfma -- `blocks` workgroups of 256 threads, each wavefront
 *   issuing `iters` x 4 independent bf16 32x32x16 matrix products (no memory
 *   traffic in the loop); out (blocks*256 fp32, device) receives one checksum
 *   per thread.  skiparse_probe_mfma_flops gives the FLOPs of one launch.
 * skiparse_probe_stream -- copies `bytes` (a multiple of 16, > 0) from src to
 *   dst (16-byte aligned, not overlapping) with 16-byte nontemporal loads and
 *   stores in a grid-stride loop over `blocks` workgroups of 256 threads.
 * One launch each on `stream`; SKIPARSE_E_* on bad arguments.
 */
int skiparse_probe_mfma(int blocks, int iters, float* out, void* stream);
double skiparse_probe_mfma_flops(int blocks, int iters);
int skiparse_probe_stream(const void* src, void* dst, int64_t bytes, int blocks, void* stream);

/* Static English text for a status code (never NULL). */
const char* skiparse_status_string(int status);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* skiparse_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKIPARSE_H */
