/*
 * moe_tqp.h -- C ABI of the MI355X (gfx950) routed-expert layer under TQP.
 *
 * The layer: a full-precision router picks k of E experts per token, each
 * expert is a SwiGLU FFN whose base weights are quantized to int4 and frozen,
 * with trained low-rank adapters on every matrix, and the k expert outputs
 * are mixed by the routing gates.  The backward produces the gradient of the
 * input and of the adapters only.
 *
 * Sources (page title, section):
 *   - skill card "Reversible Sparse MoE Single Node", Principle 3 "TQP
 *     Optimizer Strategy": base expert weights quantized and fixed, low-rank
 *     adapters carry the optimizer state.
 *   - same card, Implementation Considerations, "TQP Quantization": int8 or
 *     int4 base, full-precision trainable adapters, full-precision router.
 *   - same card, Architecture Details, and the abstract of "Reversible
 *     Foundations: Training a 120B Sparse MoE through State-Preserving
 *     Scaling": 460 routed experts under top-12 routing, 8K context.
 *   - same card, Implementation Considerations, "Reversibility": routing
 *     decisions are stateless.
 *   - same card, Related Methods: LoRA (adapter product x A B).
 * The pages fix no formats, shapes or kernels; every layout below is this
 * library's own.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) in stream order.
 *   - Arguments are validated on the host before any HIP call.  On failure
 *     the call returns a negative status, enqueues nothing and writes nothing;
 *     moe_last_error() then describes the failed check (thread-local).
 *   - Launch failures are reported as MOE_ERR_HIP.
 *   - Outputs are overwritten, never accumulated into.  Every output element
 *     is written, including zero gradients of experts that received no token.
 *   - The layer calls keep no state between calls and are re-entrant.  The
 *     one exception is the instrumentation pair moe_timer_start/stop, which
 *     holds thread-local HIP events between its start and stop calls.
 *   - Results are bitwise reproducible for identical inputs: integer
 *     histograms, scan-ordered placement, fixed-order reductions, no float
 *     atomics.
 *   - Row-major storage throughout.  "act" tensors are float32 when
 *     dims.act == MOE_F32 and bf16 (raw uint16 bit patterns) when
 *     dims.act == MOE_BF16.  Gates, logits and adapter gradients are float32.
 *
 * Shapes: T tokens, d = d_model, E experts, k experts per token, f = d_ff,
 * r = adapter rank, g = quantization group, S = T*k routed slots.
 */
#ifndef MOE_TQP_H
#define MOE_TQP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* null pointer, bad shape, bad scale          */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, group)    */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes smaller than moe_workspace_size()  */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed         */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer dimensions.  Limits: T >= 1, 1 <= k <= min(E, 32), E <= 1024,
 * group in {32, 64, 128}, d % group == 0, f % group == 0, 1 <= r <= 32,
 * S = T*k <= 2^26, d, f <= 65536, base_bits in {0, 4, 8}. */
typedef struct {
  int32_t T, d_model, n_experts, top_k, d_ff, rank, group;
  int32_t act;        /* moe_dtype */
  float lora_scale;   /* lambda in W_eff = W_hat + lambda * A B; finite */
  int32_t base_bits;  /* storage of the frozen base: 4 (int4; 0 also means 4)
                         or 8 (int8), the "Int8 or Int4" of the skill card
                         "Reversible Sparse MoE Single Node", Implementation
                         Considerations, TQP Quantization */
} moe_dims;

/* One expert matrix W[N][K] (out x in) for all E experts, frozen int4 (or
 * int8) base plus adapter.  For gate and up N = f, K = d; for down N = d,
 * K = f.
 *   q     base_bits 4: uint8 [E][N][K/2], symmetric int4, two's-complement
 *         nibbles.  Each aligned little-endian 32-bit word holds one 8-wide
 *         block k0..k7 of K; nibble slot j (bits 4j..4j+3) holds k_{2j} for
 *         j < 4 and k_{2(j-4)+1} for j >= 4.
 *         base_bits 8: uint8 [E][N][K], one two's-complement byte per value
 *         in k order.
 *   scale bf16  [E][N][K/g]: W_hat[n][c] = scale[n][c/g] * q[n][c].
 *   A     act   [E][r][K]   (out x in, like the base)
 *   B     act   [E][N][r]
 *   qt    optional (may be NULL): the base re-laid out for the input-gradient
 *         products of moe_adapter_bwd, as written by moe_pack_base_t from
 *         this q and scale.  The base is frozen under TQP, so a caller can
 *         pack it once and pass it to every backward call; with NULL the
 *         backward re-lays out the base of every expert with rows in its own
 *         workspace on each call.  Results are the same either way.  Read
 *         only by the matrix-core path (bf16, group 128, d and f multiples
 *         of 128); ignored otherwise.  16-byte aligned.
 *   qf    optional (may be NULL): the base re-laid out for the forward
 *         products of moe_expert_fwd, as written by moe_pack_base_f from
 *         this q and scale.  Same contract as qt: pack once, results
 *         identical with NULL; read only by the matrix-core path; 16-byte
 *         aligned.
 * q, A and B must be 16-byte aligned (MOE_ERR_INVALID otherwise).
 * Effective matrix: W_eff = W_hat + lambda * B A, i.e. for a row x,
 * x W_eff^T = x W_hat^T + lambda (x A^T) B^T. */
typedef struct {
  const uint8_t *q;
  const uint16_t *scale;
  const void *A;
  const void *B;
  const void *qt;
  const void *qf;
} moe_qlora;

/* Which call a workspace size is asked for. */
typedef enum {
  MOE_CALL_ROUTE = 0,
  MOE_CALL_PERMUTE = 1,
  MOE_CALL_EXPERT_FWD = 2,
  MOE_CALL_COMBINE = 3,
  MOE_CALL_ADAPTER_BWD = 4
} moe_call;

/* Flags OR-ed into the call id of moe_workspace_size: what the caller will
 * supply, so that the workspace needs no room for it.  A call checks ws_bytes
 * against the size its own arguments imply, so a workspace sized with a flag
 * is valid only for calls that do supply that.
 *   MOE_WS_SAVE_GIVEN    moe_expert_fwd with a non-NULL save buffer (without
 *                        one, the forward keeps its intermediates in the
 *                        workspace)
 *   MOE_WS_PACKED_GIVEN  moe_expert_fwd with qf set on gate, up and down, or
 *                        moe_adapter_bwd with qt set on all three (without,
 *                        the call re-lays out the base in the workspace) */
#define MOE_WS_SAVE_GIVEN 0x100
#define MOE_WS_PACKED_GIVEN 0x200

/* Router, softmax and top-k ("Reversible Sparse MoE Single Node" skill card,
 * Architecture Details: top-12 routing over 460 routed experts; Implementation
 * Considerations, TQP Quantization: the router stays full precision;
 * Reversibility: routing is a stateless function of the input).  The
 * selection order and the gate formula are this library's reading; the pages
 * state neither.  logits[t][e] = sum_c x[t][c] w_router[c][e]
 * + b_router[e] in float32; the k largest logits are selected under the order
 * (logit descending, expert index ascending) and written in that order to
 * topk_idx; gates[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
 * selected logits (softmax over all experts renormalised to the selected).
 * A NaN logit takes part as -inf, so topk_idx always holds k distinct
 * experts in [0, E) (the gates are then NaN where the logits are).
 *   x          act  [T][d]
 *   w_router   f32  [d][E]
 *   b_router   f32  [E] or NULL (no bias)
 *   topk_idx   i32  [T][k]     (out)
 *   gates      f32  [T][k]     (out)
 *   logits     f32  [T][E] or NULL (out, optional)
 *   ws         workspace of moe_workspace_size(MOE_CALL_ROUTE) bytes */
moe_status moe_route(const moe_dims *dims, const void *x, const float *w_router,
                     const float *b_router, int32_t *topk_idx, float *gates,
                     float *logits, void *ws, size_t ws_bytes, void *stream);

/* Expert histogram, scan and stable permutation of the S routed slots into
 * expert-contiguous order (expert ascending, token ascending within an
 * expert), so that each expert's tokens form one segment for the expert
 * products: the dispatch of each token to its top-k experts ("Reversible
 * Sparse MoE Single Node" skill card, Architecture Details, top-12 routing;
 * the pages leave the data movement open).  topk_idx should hold k distinct
 * entries in [0, E) per token, as moe_route writes them.  Other input is
 * made valid first, per token in j order (an entry outside [0, E) is clamped,
 * a repeated one becomes the lowest expert the token does not use yet), so
 * the placement stays a bijection and every access in bounds; the layer's
 * result is then that of the corrected routing.
 *   counts    i32 [E]     slots per expert (out)
 *   offsets   i32 [E+1]   exclusive scan of counts, offsets[E] = S (out)
 *   perm_src  i32 [S]     perm_src[p] = t*k + j of the slot at position p (out)
 *   slot_pos  i32 [S]     slot_pos[t*k + j] = p (out)
 *   x_perm    act [S][d] or NULL: x_perm[p] = x[perm_src[p] / k] (out)
 *   x         act [T][d]  read only when x_perm != NULL (may be NULL otherwise) */
moe_status moe_permute(const moe_dims *dims, const int32_t *topk_idx, const void *x,
                       int32_t *counts, int32_t *offsets, int32_t *perm_src,
                       int32_t *slot_pos, void *x_perm, void *ws, size_t ws_bytes,
                       void *stream);

/* Expert FFNs over the permuted rows, each expert a frozen quantized base
 * plus trained low-rank adapters ("Reversible Sparse MoE Single Node" skill
 * card, Principle 3 "TQP Optimizer Strategy": base expert weights quantized
 * and fixed, low-rank adapters on top; Implementation Considerations, TQP
 * Quantization: "Int8 or Int4" base, full-precision adapters; Related
 * Methods: LoRA).  The SwiGLU form, the int4 and int8 formats and the
 * adapter placement on all three matrices are this library's readings.  The rows are read from
 * x by token through perm_src (no x_perm argument: x is small enough to stay
 * in cache, which saves writing and reading the permuted copy).
 * For every position p with expert e
 * (offsets[e] <= p < offsets[e+1]) and input row X = x[perm_src[p] / k]:
 *   G = X Wg_hat^T + lambda (X A_g^T) B_g^T,  U likewise with the up matrix,
 *   H = silu(G) * U,   silu(z) = z / (1 + exp(-z))
 *   e_out[p] = H Wd_hat^T + lambda (H A_d^T) B_d^T
 * Arithmetic: MOE_F32 computes in float32 throughout; MOE_BF16 feeds bf16
 * operands to the matrix cores with float32 accumulation and rounds H and
 * e_out to bf16 (each once, to nearest even).
 *   x        act [T][d]
 *   offsets, perm_src as written by moe_permute (device)
 *   e_out    act [S][d] in permuted order (out)
 *   save     NULL, or moe_save_size() bytes that moe_adapter_bwd consumes
 *            (opaque: the intermediates the backward needs) (out)
 * x, e_out and save must be 16-byte aligned (MOE_ERR_INVALID otherwise). */
moe_status moe_expert_fwd(const moe_dims *dims, const void *x, const int32_t *offsets,
                          const int32_t *perm_src, moe_qlora gate, moe_qlora up,
                          moe_qlora down, void *e_out, void *save, void *ws,
                          size_t ws_bytes, void *stream);

/* moe_expert_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and validation
 * as moe_expert_fwd; its scratch is the library's own fixed device array of
 * 64 MiB, which every GPU the library runs on holds from module load to
 * process end (one copy per device, its address looked up on the first call
 * on that device).  The call allocates and frees nothing.
 *   - The scratch a call needs is what moe_workspace_size(MOE_CALL_EXPERT_FWD
 *     | flags) gives for the flags its own arguments imply; above 64 MiB the
 *     call returns MOE_ERR_WORKSPACE before any HIP call.  With save and the
 *     forward-packed bases (qf) given it stays a few MB at T = 8192, E = 460;
 *     with save NULL the intermediates need about S (3 d_ff act + 3 r fp32)
 *     bytes more, and without qf the ratio tables 12 E d f / 128 bytes more.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads) race on it and give
 *     undefined results.  Calls ordered on one stream are safe.  Nothing in
 *     the array needs to start at any value. */
moe_status moe_expert_fwd_noalloc(const moe_dims *dims, const void *x, const int32_t *offsets,
                                  const int32_t *perm_src, moe_qlora gate, moe_qlora up,
                                  moe_qlora down, void *e_out, void *save, void *stream);

/* Gate-weighted combine of each token's k expert outputs (the routed mixture
 * of "Reversible Sparse MoE Single Node" skill card, Architecture Details;
 * the order of the sum is this library's, fixed so that results are
 * bitwise repeatable):
 * y[t] = sum_{j=0..k-1} gates[t][j] e_out[slot_pos[t*k+j]],
 * float32 accumulation in ascending j, one rounding to act at the end.
 *   y act [T][d] (out) */
moe_status moe_combine(const moe_dims *dims, const void *e_out, const int32_t *slot_pos,
                       const float *gates, void *y, void *ws, size_t ws_bytes,
                       void *stream);

/* Additive coupling of a reversible residual block around the layer (skill
 * card "Reversible Sparse MoE Single Node": Principle 1, reconstruct rather
 * than store activations; Pattern 1, addition/subtraction as the inverse
 * operations; Implementation Considerations, reversible residual blocks and
 * stateless routing).  With m = the layer output y for the block's other
 * stream y1 (moe_combine):
 *   sign = +1:  out = x + m   (forward:  y2 = x2 + MoE(y1))
 *   sign = -1:  out = x - m   (inverse:  x2 = y2 - MoE(y1))
 * over T * d_model values in the act dtype, float32 arithmetic with one
 * rounding.  Routing is a pure function of y1, so recomputing m in the
 * backward reproduces it bit for bit; the reconstruction of x2 is exact up
 * to the two roundings to the act dtype.  out may alias x (not m).
 * Asynchronous on `stream`. */
moe_status moe_rev_couple(const moe_dims *dims, const void *x, const void *m, void *out,
                          int32_t sign, void *stream);

/* Adapter-only backward ("Reversible Sparse MoE Single Node" skill card,
 * Principle 3 "TQP Optimizer Strategy" and Pattern 3: the quantized base is
 * fixed and only the low-rank adapters are trained, so no base gradient is
 * formed; Implementation Considerations, TQP Quantization: the router is full
 * precision -- here frozen, with the gate path still carried into dx).  Rows
 * are read from x and dy by token, as in the forward (no x_perm argument).
 * Backward of route -> expert FFNs -> combine for an upstream
 * gradient dy (loss L = sum_t <dy_t, y_t>).  The selection is held fixed; the
 * router and every base matrix are frozen (no weight gradient), but the gates
 * pass gradient to x through the router:
 *   dgamma[t][j] = <dy_t, e_out[slot_pos[t,j]]>,
 *   dl[t][j] = gamma[t][j] (dgamma[t][j] - sum_i gamma[t][i] dgamma[t][i]),
 *   dx[t] = sum_j dl[t][j] w_router[:, e_{t,j}]  +  sum_j dX_expert(t, j)
 * with, per expert, Z = X A^T of each matrix and dO = gamma * dy on its rows:
 *   dB_d = lambda dO^T Z_d, dZ_d = lambda dO B_d, dA_d = dZ_d^T H,
 *   dH = dO Wd_hat + dZ_d A_d,  dG = dH U s (1 + G (1 - s)), dU = dH G s,
 *   s = sigmoid(G); dB_g = lambda dG^T Z_g, dZ_g = lambda dG B_g,
 *   dA_g = dZ_g^T X (likewise up), dX = dG Wg_hat + dU Wu_hat + dZ_g A_g
 *   + dZ_u A_u.
 * Inputs are those of the forward calls; save must hold what moe_expert_fwd
 * wrote for the same inputs.
 *   dy   act [T][d];  dx act [T][d] (out)
 *   dA_gate, dA_up f32 [E][r][d]; dB_gate, dB_up f32 [E][f][r];
 *   dA_down f32 [E][r][f]; dB_down f32 [E][d][r]  (out, layouts of A and B) */
moe_status moe_adapter_bwd(const moe_dims *dims, const void *dy, const void *x,
                           const int32_t *topk_idx, const float *gates,
                           const int32_t *offsets, const int32_t *perm_src,
                           const int32_t *slot_pos, const float *w_router,
                           moe_qlora gate, moe_qlora up, moe_qlora down,
                           const void *e_out, const void *save, void *dx,
                           float *dA_gate, float *dB_gate, float *dA_up, float *dB_up,
                           float *dA_down, float *dB_down, void *ws, size_t ws_bytes,
                           void *stream);

/* Transposed packing of one frozen base matrix for the backward (the qt
 * field of moe_qlora).  The input-gradient products reduce over the storage
 * rows N of the base, so their int4 operand must be packed along N: for
 * every expert e, block of 64 storage rows n0 and column c, 32 bytes hold
 * q[e][n0 .. n0+63][c] in the word order of the forward layout, and the
 * scales follow as float32 [E][K/128][N] (K of the matrix).  An int8 base
 * (q = 16 h + l, h = q >> 4, l = q & 15) is packed as two int4 planes
 * stacked along N: 2N rows, the first N holding h with scales 16 s, the next
 * N holding l - 8 with scales s (twice the int4 size).  The backward
 * products are those of moe_adapter_bwd (skill card "Reversible Sparse MoE
 * Single Node", Principle 3: the base is frozen, only the adapters train).
 *   matrix  MOE_MAT_GATE_UP (q [E][f][d/2], scale [E][f][d/128]) or
 *           MOE_MAT_DOWN (q [E][d][f/2], scale [E][d][f/128])
 *   packed  device buffer of moe_pack_base_t_size() bytes, 16-byte aligned
 *           (out; caller-owned)
 * Only the matrix-core path has this layout: other dims give
 * MOE_ERR_UNSUPPORTED.  Asynchronous on `stream`. */
typedef enum { MOE_MAT_GATE_UP = 0, MOE_MAT_DOWN = 1 } moe_matrix;
moe_status moe_pack_base_t_size(const moe_dims *dims, size_t *bytes);
moe_status moe_pack_base_t(const moe_dims *dims, int32_t matrix, const uint8_t *q,
                           const uint16_t *scale, void *packed, size_t packed_bytes,
                           void *stream);

/* Stage-major packing of one frozen base matrix for the forward (the qf
 * field of moe_qlora).  The forward products reduce over K in steps of 64,
 * each step reading 32 bytes of every output column; packed, one step of
 * one expert is a contiguous run: for every expert e, block of 64 columns of
 * K k0 and storage row n, 32 bytes hold q[e][n][k0/2 .. k0/2+31] unchanged
 * (layout [E][K/64][N][32 B], the byte count of q).  An int8 base is packed
 * as two int4 planes along K (2K columns: h = q >> 4, then l - 8 with
 * l = q & 15, in the int4 word order), with the plane scales 16 s and s in
 * the ratio table below (2 K/128 groups); the byte count of q again.  The float32 table of
 * group-scale ratios the forward applies follows, [E][K/128][N]: entry g >= 1
 * of column n is s'[n][g-1] / s'[n][g] and entry 0 is s'[n][K/128-1], where
 * s' is the bf16 scale with magnitudes below the column's floor raised to
 * that floor; the floor is 2^-24 times the column's largest |scale|, and at
 * least 2^-100 (so no ratio exceeds 2^24).  The
 * products are those of moe_expert_fwd (skill card "Reversible Sparse MoE
 * Single Node", Principle 3: the quantized base is fixed, so it is packed
 * once).
 *   matrix  MOE_MAT_GATE_UP (q [E][f][d/2], scale [E][f][d/128]) or
 *           MOE_MAT_DOWN (q [E][d][f/2], scale [E][d][f/128])
 *   packed  device buffer of moe_pack_base_f_size() bytes, 16-byte aligned
 *           (out; caller-owned); must not overlap q
 * Only the matrix-core path has this layout: other dims give
 * MOE_ERR_UNSUPPORTED.  Asynchronous on `stream`. */
moe_status moe_pack_base_f_size(const moe_dims *dims, size_t *bytes);
moe_status moe_pack_base_f(const moe_dims *dims, int32_t matrix, const uint8_t *q,
                           const uint16_t *scale, void *packed, size_t packed_bytes,
                           void *stream);

/* Few -> many expert growth ("Reversible Sparse MoE Single Node" skill
 * card, Principle 2 "State-Preserving Growth": few to many, duplicate experts
 * and reinitialise routing).  Grown expert e * factor + c (c = 0 ..
 * factor-1) is a copy of expert e, so every per-expert tensor of the layer
 * (q, scale, A, B of each matrix) is grown by moe_grow_copy and the router
 * by moe_grow_router; the grown layer has n_experts * factor experts and,
 * to compute the same function, top_k * factor experts per token (then the
 * factor copies of each selected expert tie, are all selected and share its
 * gate).  Limits: factor >= 1, n_experts * factor <= 1024.
 *   moe_grow_copy:   src holds n_experts blocks of block_bytes; dst
 *                    (n_experts * factor blocks, caller-owned) must not
 *                    overlap src.
 *   moe_grow_router: w_router [d][E] f32 -> w_out [d][E factor]; column
 *                    e factor + c is column e, moved for c >= 1 by
 *                    noise_scale * noise[i][e factor + c] (noise [d][E factor]
 *                    f32, caller-drawn; NULL or noise_scale 0 keeps every
 *                    copy exact), in float32 with one rounding; b_router [E]
 *                    (or NULL) -> b_out [E factor] copied.
 * Asynchronous on `stream`. */
moe_status moe_grow_copy(const void *src, void *dst, int64_t block_bytes, int32_t n_experts,
                         int32_t factor, void *stream);
moe_status moe_grow_router(int32_t d, int32_t n_experts, int32_t factor, const float *w_router,
                           const float *b_router, const float *noise, float noise_scale,
                           float *w_out, float *b_out, void *stream);

/* Adapter optimizer step: AdamW on one float32 tensor of n elements (call it
 * once per adapter tensor: A and B of gate, up and down).  The optimizer
 * state lives on the adapters only, the quantized base being fixed (skill
 * card "Reversible Sparse MoE Single Node", Principle 3 "TQP Optimizer
 * Strategy" and Pattern 3).  The pages name no optimizer; this library reads
 * it as AdamW ("Decoupled Weight Decay Regularization", Loshchilov and
 * Hutter): with t = step,
 *   m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2,
 *   master <- master - lr ( (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *                           + weight_decay master )
 * in float32 (the bias corrections 1 - beta^t are formed in double on the
 * host).  Elementwise; master, m, v are updated in place.
 *   master  f32 [n]  float32 master copy of the adapter (in/out)
 *   grad    f32 [n]  its gradient, e.g. dA_gate of moe_adapter_bwd (layouts
 *                    of A and B, so any flat order works)
 *   m, v    f32 [n]  first and second moments (in/out; zero before step 1)
 *   param   NULL, or [n] in param_dtype (MOE_F32 or MOE_BF16, rounded to
 *           nearest even): a copy of the new master, e.g. the act-dtype
 *           adapter that moe_expert_fwd reads (out)
 * The four float32 buffers must be distinct (param may not alias them).
 * Validation: step >= 1, beta1, beta2 in [0, 1), eps finite and > 0, lr and
 * weight_decay finite, n >= 0 (n = 0 enqueues nothing). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t step;
} moe_adamw_hparams;
moe_status moe_adamw_step(const moe_adamw_hparams *h, int64_t n, float *master,
                          const float *grad, float *m, float *v, void *param,
                          int32_t param_dtype, void *stream);

/* Instrumentation, not part of the method: time every launch of one internal
 * kernel with a pair of HIP events recorded on the launch stream around it.
 * moe_timer_start arms the calling thread for `tag` (one of moe_kernel_tag;
 * at most 4096 launches are recorded); moe_timer_stop waits for the recorded
 * events, returns the summed milliseconds and the number of launches, and
 * disarms.  Events are created on the first use and reused; the state is
 * thread-local. */
typedef enum {
  MOE_KT_ROUTER_LOGITS = 0, /* router GEMM (float32 matrix cores)          */
  MOE_KT_ROUTER_TOPK = 1,   /* partial sum, top-k, softmax                  */
  MOE_KT_PERMUTE = 2,       /* scatter of the permutation                   */
  MOE_KT_GATEUP = 3,        /* gate/up expert GEMM with SwiGLU epilogue     */
  MOE_KT_DOWN = 4,          /* down expert GEMM                             */
  MOE_KT_COMBINE = 5,       /* gate-weighted combine                        */
  MOE_KT_GATE_GRAD = 6,     /* gate / router-input gradient (dO, or on the
                               matrix-core path the final sum of dX)       */
  MOE_KT_BWD_DOWN = 7,      /* dH = dO W_d + dZ_d A_d^T (and SwiGLU bwd)    */
  MOE_KT_BWD_GATEUP = 8,    /* dX_perm = dG W_g + dU W_u + ...              */
  MOE_KT_COUNT = 9
} moe_kernel_tag;
moe_status moe_timer_start(int32_t tag);
moe_status moe_timer_stop(float *total_ms, int32_t *launches);

/* Host-only queries; they validate dims like the calls do. */
moe_status moe_workspace_size(const moe_dims *dims, int32_t call, size_t *bytes);
moe_status moe_save_size(const moe_dims *dims, size_t *bytes);
const char *moe_status_string(int32_t status);
const char *moe_last_error(void);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_TQP_H */
