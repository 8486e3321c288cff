/*
 * moe_ffn.h - C ABI of the local Mixture-of-Experts FFN forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The computation (ruDNN user guide, "3. MoE workflow"):
 *   logits -> fp32 softmax over all experts -> top-k -> compact dispatch ->
 *   bias-free SwiGLU experts -> weighted combine restoring token order,
 * plus the fused combine + residual Add + RMSNorm epilogue of the CANN
 * operator aclnnMoeDistributeCombineAddRmsNormV2 ("function description",
 * formula), restricted to one device.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are dense, row-major, caller-owned DEVICE memory on the device
 *    of `stream` (e.g. allocated by PyTorch). The library allocates nothing
 *    and keeps no state between calls.
 *  - Scratch memory is caller-provided: each call that needs it takes
 *    (`ws`, `ws_bytes`) and has a `*_workspace_size` query returning the
 *    bytes it needs (the two-phase "get workspace size, then execute on a
 *    stream" convention of the CANN operator pages). `ws` must be 256-byte
 *    aligned. Concurrent calls need distinct workspaces.
 *  - Every call validates its arguments on the host before enqueueing
 *    anything; on error nothing is enqueued and a status is returned
 *    (ruDNN user guide, "3. MoE workflow": invalid shapes, dtypes or other
 *    arguments are errors; "6. Calling MoE": shape, dtype or device
 *    mismatches are errors). On success the work is enqueued on `stream`
 *    and the call returns without synchronising the host.
 *  - T = 0 is a successful no-op. NaN / +inf / -inf logits are data, not
 *    errors (routing contract, below).
 *  - Sizes are int64_t; T*top_k must fit in int32; E <= 1024.
 *  - Row lengths H and I must be multiples of 8 elements (16 bytes of
 *    bf16/f16; fp32 tensors are also read in 8-element steps).
 *  - bf16 / f16 expert GEMMs (every call that runs them: the experts calls,
 *    the forward calls and the experts' training forward) address their
 *    operands with 32-bit byte offsets. They return UNSUPPORTED, before
 *    enqueueing anything, unless each of these is below 2^31 bytes: the
 *    token rows the gate/up GEMM reads (x_disp, or x when read through a
 *    map: a_rows * H * b), h (rows * I * b), one expert's weight matrix
 *    (I * H * b), and 256 * max(H, 2 * I) * 4. (b = 2; fp32 experts use
 *    64-bit addressing and have no such limit.)
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_F16 = 1,
  MOE_BF16 = 2
} moe_dtype;

typedef enum moe_status {
  MOE_SUCCESS = 0,
  MOE_ERROR_NULL_POINTER = 1, /* a required pointer is NULL */
  MOE_ERROR_SHAPE = 2,        /* negative or inconsistent sizes */
  MOE_ERROR_DTYPE = 3,        /* unknown dtype, or x/weights dtypes differ */
  MOE_ERROR_ARGUMENT = 4,     /* top_k outside [1, E]; eps not finite or <= 0;
                                 an output overlaps an input or another output */
  MOE_ERROR_DEVICE = 5,       /* a pointer is not device memory of the stream's device */
  MOE_ERROR_WORKSPACE = 6,    /* workspace NULL, misaligned or too small */
  MOE_ERROR_UNSUPPORTED = 7,  /* E > 1024, T*top_k > INT32_MAX, H or I not a multiple of 8,
                                 a row of H elements longer than INT32_MAX bytes, or a bf16 /
                                 f16 expert GEMM operand of 2^31 bytes or more (see below) */
  MOE_ERROR_HIP = 8           /* a HIP launch or query failed */
} moe_status;

/* Human-readable name of a status (static string, never NULL). */
const char* moe_status_string(moe_status s);

/*
 * moe_route - routing plan from logits.
 * Passage: ruDNN user guide, "4. Routing contract".
 *   logits   [T, E], dtype logits_dt (F32, F16 or BF16), read only.
 *   For each token: p = softmax over all E experts, computed in fp32; the
 *   top_k experts by p are selected, largest first, equal p favouring the
 *   lower expert id. With renormalize != 0 the selected p are divided by
 *   their sum. Weights are then converted to logits_dt.
 *   A row that contains a NaN, contains +inf, or is entirely -inf keeps NaN
 *   weights (no uniform fallback); its indices are 0..top_k-1 (NaNs tie, and
 *   ties favour the lower id).
 *   indices  [T, top_k] uint32, written.
 *   weights  [T, top_k] logits_dt, written.
 * Errors: ARGUMENT if top_k not in [1, E]; UNSUPPORTED if E > 1024.
 */
moe_status moe_route(const void* logits, moe_dtype logits_dt, int64_t T, int64_t E,
                     int64_t top_k, int renormalize, uint32_t* indices, void* weights,
                     hipStream_t stream);

/*
 * moe_dispatch - compact grouping of tokens by expert, no capacity drop.
 * Passage: ruDNN user guide, "5. Expert weights and dispatch" (no token is
 * dropped to enforce a capacity; a saved map restores token order).
 *   indices        [T, top_k] uint32 expert ids (e.g. from moe_route), read.
 *   x              [T, H] dtype dt, read; may be NULL only if x_disp is NULL.
 *   x_disp         [T*top_k, H] dtype dt, written: rows grouped by expert;
 *                  may be NULL (maps only).
 *   expert_offsets [E+1] int32, written: rows of expert e are
 *                  expert_offsets[e] .. expert_offsets[e+1]-1.
 *   slot_of_row    [T*top_k] int32, written: flat slot t*top_k+j held by
 *                  dispatched row r (only the first expert_offsets[E] rows).
 *   row_of_slot    [T*top_k] int32, written: the inverse map (-1 for a slot
 *                  whose expert id is >= E; such slots are not dispatched).
 *   Order inside an expert: increasing flat slot (deterministic; the pages
 *   leave this order free).
 *   ws / ws_bytes  scratch, at least moe_dispatch_workspace_size(T, top_k, E).
 */
moe_status moe_dispatch(const uint32_t* indices, int64_t T, int64_t top_k, int64_t E,
                        const void* x, moe_dtype dt, int64_t H, void* x_disp,
                        int32_t* expert_offsets, int32_t* slot_of_row, int32_t* row_of_slot,
                        void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_dispatch_workspace_size(int64_t T, int64_t top_k, int64_t E);

/*
 * moe_dispatch_masked - moe_dispatch with an activity mask.
 * Passages: ruDNN user guide, "5. Expert weights and dispatch"; the mask is
 * the xActiveMaskOptional input of aclnnMoeDistributeCombineAddRmsNormV2
 * (a per-token flag, or one flag per (token, expert slot); a token whose
 * flags are all off takes no part).
 *   active     NULL (mask_dims 0: every slot active), or uint8 [T]
 *              (mask_dims 1: one flag per token) or [T, top_k] (mask_dims 2:
 *              one flag per slot); nonzero = active. Any pattern is accepted
 *              (the page's "active tokens first" rule serves its
 *              communication layout, not this computation).
 *   Slots that are inactive or whose id is >= E are not dispatched
 *   (row_of_slot = -1); ids >= E may name special experts handled by
 *   moe_combine_special. top_k may exceed E. Other arguments, results and
 *   errors as moe_dispatch; ARGUMENT if mask_dims is not 0..2 or does not
 *   match whether active is given.
 */
moe_status moe_dispatch_masked(const uint32_t* indices, const uint8_t* active, int mask_dims,
                               int64_t T, int64_t top_k, int64_t E, const void* x, moe_dtype dt,
                               int64_t H, void* x_disp, int32_t* expert_offsets,
                               int32_t* slot_of_row, int32_t* row_of_slot, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * moe_experts_forward_dispatched - bias-free SwiGLU experts on dispatched rows.
 * Passages: ruDNN user guide, "3. MoE workflow" (SwiGluExperts::new builds
 * bias-free expert weights; forward_dispatched computes the dispatched
 * tokens) and "5. Expert weights and dispatch" (layouts).
 *   x_disp         [rows, H] dtype dt, read (rows grouped by expert).
 *   expert_offsets [E+1] int32 device array from moe_dispatch, read on the
 *                  device (counts never return to the host).
 *   rows           host upper bound of expert_offsets[E] (normally T*top_k).
 *   w_gate, w_up   [E, I, H] dtype dt;  w_down [E, H, I] dtype dt.
 *   For every dispatched row r of expert e:
 *     h = SiLU(W_gate[e] x_r) * (W_up[e] x_r)    (length I, stored in dt)
 *     expert_out[r] = W_down[e] h                (length H, stored in dt)
 *   with SiLU(g) = g / (1 + exp(-g)) and fp32 accumulation.
 *   expert_out     [rows, H] dtype dt, written for rows < expert_offsets[E].
 *   ws / ws_bytes  scratch, at least moe_experts_workspace_size(...).
 * dt: BF16 and F16 run on the matrix cores; F32 on the vector ALUs.
 */
moe_status moe_experts_forward_dispatched(const void* x_disp, const int32_t* expert_offsets,
                                          int64_t rows, int64_t E, int64_t H, int64_t I,
                                          const void* w_gate, const void* w_up,
                                          const void* w_down, moe_dtype dt, void* expert_out,
                                          void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_experts_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I, moe_dtype dt);

/*
 * moe_experts_gate_up / moe_experts_down - the two halves of
 * moe_experts_forward_dispatched, for callers that want h or time the GEMMs
 * separately. Same passages and arithmetic.
 *   moe_experts_gate_up:  h[r] = SiLU(W_gate[e] a_r) * (W_up[e] a_r), h [rows, I] dt.
 *     With row_map == NULL, a_r is row r of x (x = x_disp, [rows, H]).
 *     With row_map != NULL, a_r is row row_map[r] / map_div of x (x = the
 *     token matrix [ceil(rows/map_div), H]); pass slot_of_row from
 *     moe_dispatch and map_div = top_k to read tokens without materialising
 *     x_disp. Map entries are clamped to the rows of x.
 *   moe_experts_down:  expert_out[r] = W_down[e] h[r], expert_out [rows, H] dt.
 *   ws / ws_bytes: at least moe_experts_gemm_workspace_size(rows, E, H, I, dt)
 *   (the device-built tile list, and for the down GEMM possibly fp32
 *   split-K partial sums); one workspace per in-flight call.
 * Errors: ARGUMENT if row_map is given and map_div is not in [1, rows].
 */
moe_status moe_experts_gate_up(const void* x, const int32_t* row_map, int64_t map_div,
                               const int32_t* expert_offsets, int64_t rows, int64_t E, int64_t H,
                               int64_t I, const void* w_gate, const void* w_up, moe_dtype dt,
                               void* h, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_experts_down(const void* h, const int32_t* expert_offsets, int64_t rows, int64_t E,
                            int64_t H, int64_t I, const void* w_down, moe_dtype dt,
                            void* expert_out, void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_experts_gemm_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                       moe_dtype dt);

/*
 * moe_combine - restore token order and merge expert outputs.
 * Passage: ruDNN user guide, "6. Calling MoE" (combine uses the dispatch map
 * to restore token order and merges expert outputs with the routing weights).
 *   out[t] = sum_{j<top_k} weights[t,j] * expert_out[row_of_slot[t*top_k+j]]
 *   accumulated in fp32 in j order, stored in dt. A token with a slot whose
 *   row is -1 gets a NaN row.
 *   expert_out [rows, H] dt; row_of_slot [T*top_k] int32; weights [T, top_k]
 *   w_dt; out [T, H] dt (written).
 */
moe_status moe_combine(const void* expert_out, const int32_t* row_of_slot, const void* weights,
                       moe_dtype w_dt, int64_t T, int64_t top_k, int64_t H, moe_dtype dt,
                       void* out, hipStream_t stream);

/*
 * moe_forward - the whole local forward: route -> dispatch -> experts ->
 * combine, on one stream, no host synchronisation.
 * Passage: ruDNN user guide, "6. Calling MoE" (forward(input, logits,
 * options) takes precomputed logits; it does not run the model's gate
 * projection or load weight files).
 *   x [T, H] dt; logits [T, E] logits_dt; weights as in
 *   moe_experts_forward_dispatched; out [T, H] dt (written).
 *   indices_out [T, top_k] uint32 and weights_out [T, top_k] logits_dt are
 *   optional copies of the routing plan (NULL to skip).
 *   offsets_out [E+1] int32, optional (NULL to skip): the per-expert row
 *   offsets of the dispatch (expert_offsets of moe_dispatch), so a caller can
 *   read the expert loads without a second dispatch.
 *   ws / ws_bytes scratch, at least moe_forward_workspace_size(...).
 *   stage_events: NULL, or 6 caller-created HIP events recorded on `stream`
 *   before route, after route, after dispatch, after the gate/up GEMM, after
 *   the down GEMM and after the combine (per-stage timing).
 */
moe_status moe_forward(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                       int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                       const void* w_gate, const void* w_up, const void* w_down, moe_dtype dt,
                       void* out, uint32_t* indices_out, void* weights_out,
                       int32_t* offsets_out, void* ws, size_t ws_bytes,
                       hipEvent_t* stage_events, hipStream_t stream);
size_t moe_forward_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k,
                                  moe_dtype dt, moe_dtype logits_dt);

/*
 * moe_forward_noalloc - moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument; the call uses a scratch array the
 * library holds in its own device memory, MOE_NOALLOC_SCRATCH_BYTES (64 MiB)
 * on every device it runs on, kept until the process ends. It calls no
 * allocating routine.
 *   Arguments, results and errors as moe_forward (outputs stay caller-owned),
 *   plus WORKSPACE when moe_forward_workspace_size(T, H, I, E, top_k, dt,
 *   logits_dt) exceeds MOE_NOALLOC_SCRATCH_BYTES (nothing is enqueued); that
 *   holds decode and serving batches (e.g. 16 tokens of E 128, top-8, H 4096,
 *   I 1536 need about 2 MB), not the large prefill batches.
 *   Every call on one device shares that device's array: calls on one stream
 *   are ordered, but calls that may run at the same time on one device (other
 *   streams, other host threads) race on it. The array keeps the last call's
 *   contents; nothing in it needs to start at zero.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                               int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                               const void* w_gate, const void* w_up, const void* w_down,
                               moe_dtype dt, void* out, uint32_t* indices_out, void* weights_out,
                               int32_t* offsets_out, hipEvent_t* stage_events, hipStream_t stream);

/*
 * moe_route_sigmoid_grouped - grouped-limited sigmoid routing with an
 * optional correction bias.
 * Passage: ruDNN user guide, "10. Grouped-limited sigmoid MoE routing"
 * (route_sigmoid_grouped and GroupRoutingOptions).
 *   logits   [T, E], dtype logits_dt (F32, F16 or BF16), read only.
 *   bias     [E] fp32 correction bias, read only; NULL = no bias.
 *   For each token: s = sigmoid(z) in fp32 and c = s + bias. The E experts
 *   form `groups` equal contiguous groups (expert e in group e / (E/groups));
 *   a group's score is the sum of its two largest c when group_top_two != 0,
 *   else its largest c. The `selected_groups` best groups are kept (equal
 *   scores: lower group first); among their experts the top_k largest c are
 *   selected, largest first, equal c favouring the lower id. The bias only
 *   steers the selection: weights are the selected s, divided by their sum
 *   when renormalize != 0, then multiplied by scale and converted to
 *   logits_dt. A row whose c contains a NaN gets indices 0..top_k-1 and NaN
 *   weights (the convention of moe_route).
 *   indices  [T, top_k] uint32, written.  weights [T, top_k] logits_dt, written.
 * Errors: ARGUMENT unless 1 <= groups <= 128, groups divides E,
 *   1 <= selected_groups <= groups, 1 <= top_k <= min(64, selected_groups *
 *   E / groups), E / groups >= 2 when group_top_two, scale finite and > 0;
 *   UNSUPPORTED if E > 1024.
 */
moe_status moe_route_sigmoid_grouped(const void* logits, moe_dtype logits_dt, int64_t T, int64_t E,
                                     const float* bias, int64_t top_k, int64_t groups,
                                     int64_t selected_groups, int group_top_two, int renormalize,
                                     float scale, uint32_t* indices, void* weights,
                                     hipStream_t stream);

/*
 * moe_forward_sigmoid_grouped - moe_forward with the grouped-limited sigmoid
 * router of moe_route_sigmoid_grouped in place of the softmax router.
 * Passage: ruDNN user guide, "10. Grouped-limited sigmoid MoE routing"
 * (SwiGluExperts::forward_sigmoid_grouped: routing, dispatch, experts and
 * combine in one call; shared experts and residuals stay with the caller).
 *   Arguments as in moe_forward, plus bias / groups / selected_groups /
 *   group_top_two / scale as in moe_route_sigmoid_grouped (same checks).
 *   Workspace: moe_forward_workspace_size(T, H, I, E, top_k, dt, logits_dt).
 */
moe_status moe_forward_sigmoid_grouped(const void* x, const void* logits, moe_dtype logits_dt,
                                       int64_t T, int64_t H, int64_t I, int64_t E,
                                       const float* bias, int64_t top_k, int64_t groups,
                                       int64_t selected_groups, int group_top_two,
                                       int renormalize, float scale, const void* w_gate,
                                       const void* w_up, const void* w_down, moe_dtype dt,
                                       void* out, uint32_t* indices_out, void* weights_out,
                                       int32_t* offsets_out, void* ws, size_t ws_bytes,
                                       hipEvent_t* stage_events, hipStream_t stream);

/*
 * moe_combine_add_rmsnorm - combine fused with the shared-expert term, the
 * residual Add and RMSNorm.
 * Passages: aclnnMoeDistributeCombineAddRmsNormV2, "function description"
 * (formula) and parameter list (yOut, rstdOut, xOut); ruDNN user guide,
 * "7. LayerNorm, RMSNorm and Softmax" (fp32 statistics and affine math,
 * F32 gamma, output in the input dtype, eps finite and > 0).
 *   c[t]    = sum_j weights[t,j] * (expert_out[row_of_slot[t*k+j]] + shared[t])
 *             (shared may be NULL: term omitted)
 *   x[t]    = c[t] + residual[t]
 *   rstd[t] = 1 / sqrt(mean_H(x[t]^2) + eps)
 *   y[t]    = x[t] * rstd[t] * gamma
 *   all in fp32; x_out = x and y stored in dt, rstd in fp32.
 *   expert_out [rows, H] dt; shared, residual [T, H] dt; gamma [H] fp32;
 *   y, x_out [T, H] dt (written); rstd [T] fp32 (written).
 * Errors: ARGUMENT if eps is not finite or <= 0; UNSUPPORTED if H > 32768.
 */
moe_status moe_combine_add_rmsnorm(const void* expert_out, const int32_t* row_of_slot,
                                   const void* weights, moe_dtype w_dt, const void* shared,
                                   const void* residual, const float* gamma, float eps,
                                   int64_t T, int64_t top_k, int64_t H, moe_dtype dt,
                                   void* y, void* x_out, float* rstd, hipStream_t stream);

/*
 * moe_combine_special - combine with special experts and an activity mask.
 * Passage: aclnnMoeDistributeCombineAddRmsNormV2, "function description"
 * (special experts: Moe(oriX) = 0 for zero experts, oriX for copy experts,
 * constExpertAlpha1 * oriX + constExpertAlpha2 * constExpertV for constant
 * experts) and its parameters zeroExpertNum / copyExpertNum /
 * constExpertNum, oriXOptional, constExpertAlpha1Optional /
 * constExpertAlpha2Optional / constExpertVOptional, xActiveMaskOptional and
 * sharedExpertXOptional.
 *   For each token t: out[t] = sum over active slots j of
 *     weights[t,j] * (m_j + shared[t])  (shared may be NULL: term omitted)
 *   with e = indices[t,j] and
 *     e < E                                expert_out[row_of_slot[t*k+j]]
 *     E <= e < E+zero_num                  0
 *     next copy_num ids                    ori_x[t]
 *     next const_num ids (constant q)      const_alpha1[q]*ori_x[t] + const_alpha2[q]*const_v[q]
 *   Any other id, or a real-expert slot that was not dispatched, makes the
 *   token's row NaN; a token with no active slot combines to 0. fp32
 *   arithmetic, out rounded once to dt.
 *   expert_out [rows, H] dt; row_of_slot [T*top_k] int32 (from moe_dispatch
 *   or moe_dispatch_masked with the same mask); indices [T, top_k] uint32;
 *   weights [T, top_k] w_dt; ori_x [T, H] dt (needed when copy_num or
 *   const_num > 0); const_alpha1, const_alpha2 [const_num] dt; const_v
 *   [const_num, H] dt; active / mask_dims as in moe_dispatch_masked;
 *   out [T, H] dt (written).
 * Errors: ARGUMENT for negative counts, E + counts > 2^31 - 1 or a bad mask
 *   description; NULL_POINTER when a needed input is missing; UNSUPPORTED if
 *   H is not a multiple of 8 or exceeds 32768.
 */
moe_status moe_combine_special(const void* expert_out, const int32_t* row_of_slot,
                               const uint32_t* indices, const void* weights, moe_dtype w_dt,
                               int64_t T, int64_t top_k, int64_t H, moe_dtype dt, int64_t E,
                               int64_t zero_num, int64_t copy_num, int64_t const_num,
                               const void* ori_x, const void* const_alpha1,
                               const void* const_alpha2, const void* const_v,
                               const uint8_t* active, int mask_dims, const void* shared,
                               void* out, hipStream_t stream);

/*
 * moe_combine_add_rmsnorm_special - moe_combine_special followed by the
 * residual Add and RMSNorm of moe_combine_add_rmsnorm (the whole
 * aclnnMoeDistributeCombineAddRmsNormV2 formula with special experts and the
 * activity mask): x = combined + residual, rstd = 1/sqrt(mean(x^2) + eps),
 * y = x * rstd * gamma; x_out = x and y in dt, rstd fp32. A token with no
 * active slot gets x = residual.
 * Errors: as moe_combine_special, plus ARGUMENT if eps is not finite or <= 0.
 */
moe_status moe_combine_add_rmsnorm_special(
    const void* expert_out, const int32_t* row_of_slot, const uint32_t* indices,
    const void* weights, moe_dtype w_dt, int64_t T, int64_t top_k, int64_t H, moe_dtype dt,
    int64_t E, int64_t zero_num, int64_t copy_num, int64_t const_num, const void* ori_x,
    const void* const_alpha1, const void* const_alpha2, const void* const_v,
    const uint8_t* active, int mask_dims, const void* shared, const void* residual,
    const float* gamma, float eps, void* y, void* x_out, float* rstd, hipStream_t stream);

/*
 * moe_experts_forward_dispatched_quant - bias-free SwiGLU experts with
 * weight-only INT8 / INT4 weights, for decode-sized batches.
 * Passage: aclnnFFN, "Formula", pseudo-quantization scenario
 * (y = activation(x * ((W1 + antiquantOffset1) * antiquantScale1)) *
 * ((W2 + antiquantOffset2) * antiquantScale2), here with the SwiGLU of
 * moe_experts_forward_dispatched), and its constraints (INT8 or INT4
 * weights; per-group scales only with INT4; the group count divides both
 * input sizes; INT4 rows of even length).
 *   Weights keep the K-contiguous layout of the bf16 ones:
 *     bits = 8: w_gate, w_up [E, I, H] int8; w_down [E, H, I] int8.
 *     bits = 4: the same shapes with two values per byte along K (element
 *               k in byte k/2, low nibble first, two's complement -8..7).
 *   Each weight enters as (q + offset) * scale with
 *     scale_gate, scale_up [E, I, groups], scale_down [E, H, groups] in dt,
 *     offset_*: same shapes, or NULL for 0;
 *   group j of a row covers input channels j*K/groups .. (j+1)*K/groups - 1
 *   (groups = 1: one scale per output channel). Each weight is taken as
 *   the exact (q + offset) * scale, not rounded to dt: per group the
 *   kernels accumulate sum(x * (q + C)) and sum(x) in fp32 for a constant
 *   code shift C and add scale * sum(x * (q + C)) + (offset - C) * scale *
 *   sum(x); only the two GEMMs' results are rounded to dt.
 *   Other arguments as moe_experts_forward_dispatched; workspace:
 *   moe_experts_quant_workspace_size(rows, E, H, I, dt) (holds h).
 * Errors: ARGUMENT if bits is not 8 or 4, groups < 1 or does not divide H
 *   and I, or groups > 1 with bits = 8; UNSUPPORTED for dt F32, for
 *   groups > 1 unless H/groups and I/groups are multiples of 128, for
 *   rows > 4 * E (this path streams weights for decode-sized batches), and
 *   when one expert's codes or 4*E activation rows exceed 2^31 bytes.
 */
moe_status moe_experts_forward_dispatched_quant(
    const void* x_disp, const int32_t* expert_offsets, int64_t rows, int64_t E, int64_t H, int64_t I,
    const void* w_gate, const void* w_up, const void* w_down, int bits, int64_t groups,
    const void* scale_gate, const void* scale_up, const void* scale_down, const void* offset_gate,
    const void* offset_up, const void* offset_down, moe_dtype dt, void* expert_out, void* ws,
    size_t ws_bytes, hipStream_t stream);
size_t moe_experts_quant_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                        moe_dtype dt);

/*
 * moe_forward_quant - moe_forward with the weight-only quantised experts of
 * moe_experts_forward_dispatched_quant (same weight, scale and offset
 * arguments and checks; rows = T * top_k). Passages: ruDNN user guide, "6.
 * Calling MoE"; aclnnFFN, pseudo-quantization scenario.
 * Workspace: moe_forward_workspace_size(T, H, I, E, top_k, dt, logits_dt).
 */
moe_status moe_forward_quant(const void* x, const void* logits, moe_dtype logits_dt, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t top_k, int renormalize,
                             const void* w_gate, const void* w_up, const void* w_down, int bits,
                             int64_t groups, const void* scale_gate, const void* scale_up,
                             const void* scale_down, const void* offset_gate,
                             const void* offset_up, const void* offset_down, moe_dtype dt,
                             void* out, uint32_t* indices_out, void* weights_out,
                             int32_t* offsets_out, void* ws, size_t ws_bytes,
                             hipEvent_t* stage_events, hipStream_t stream);

/* ===================== first-order training ===================== */
/*
 * Passage for everything below: ruDNN user guide, "12. MoE first-order
 * training" (router weights for a fixed selection and their backward;
 * forward_dispatched_training keeping a cache; the backward order
 * combine_backward -> expert backward -> dispatch_backward -> router
 * backward; weight gradients and dweights in FP32). Gradients are taken with
 * the selection held fixed: top-k and group decisions are not differentiated.
 */
typedef enum moe_scoring {
  MOE_SCORE_SOFTMAX = 0, /* softmax over all E experts, gathered at the indices */
  MOE_SCORE_SIGMOID = 1  /* sigmoid of the selected logits */
} moe_scoring;

typedef enum moe_index_dtype {
  MOE_IDX_U32 = 0,
  MOE_IDX_I32 = 1,
  MOE_IDX_I64 = 2
} moe_index_dtype;

/*
 * moe_router_weights - weights of a fixed selection (selected_router_weights).
 *   logits   [T, E] logits_dt, read; indices [T, top_k] idx_dt, read.
 *   a[t,j] = softmax(logits[t])[idx] (fp32, over all E) or
 *            sigmoid(logits[t, idx]); repeated indices gather again.
 *   normalize != 0: a[t,j] /= sum_j a[t,j]. Then weights = a * scale.
 *   weights  [T, top_k] fp32, written. A row holding an index outside
 *            [0, E) is NaN throughout (nothing is read out of bounds).
 * Errors: ARGUMENT if top_k not in [1, min(E, 64)], scoring unknown, or
 *   scale not finite and > 0; DTYPE for an unknown idx_dt.
 */
moe_status moe_router_weights(const void* logits, moe_dtype logits_dt, const void* indices,
                              moe_index_dtype idx_dt, int64_t T, int64_t E, int64_t top_k,
                              moe_scoring scoring, int normalize, float scale, float* weights,
                              hipStream_t stream);

/*
 * moe_router_backward - d loss / d logits for the weights of
 * moe_router_weights (selected_router_backward), same arguments plus
 *   grad_weights [T, top_k] fp32, read;
 *   grad_logits  [T, E] logits_dt, written (every element). Unselected
 *   experts receive the softmax coupling term (no normalize) or 0. A row
 *   with an invalid index, and a softmax row whose logits contain NaN or
 *   +inf or are all -inf, is NaN throughout.
 */
moe_status moe_router_backward(const void* logits, moe_dtype logits_dt, const void* indices,
                               moe_index_dtype idx_dt, const float* grad_weights, int64_t T,
                               int64_t E, int64_t top_k, moe_scoring scoring, int normalize,
                               float scale, void* grad_logits, hipStream_t stream);

/*
 * moe_combine_backward - gradient of moe_combine (combine_backward).
 *   expert_out [rows, H] dt, row_of_slot [T*top_k], weights [T, top_k] w_dt,
 *   grad_out [T, H] dt: read. rows (<= T*top_k) is the number of
 *   dispatched rows the two row buffers hold; every row_of_slot entry must
 *   be -1 or below it.
 *   dexpert  [rows, H] dt, written for every dispatched row:
 *            dexpert[row(t,j)] = weights[t,j] * grad_out[t].
 *   dweights [T, top_k] fp32, written: <grad_out[t], expert_out[row(t,j)]>
 *            accumulated in fp32; NaN for a slot without a row (-1).
 */
moe_status moe_combine_backward(const void* expert_out, const int32_t* row_of_slot,
                                const void* weights, moe_dtype w_dt, const void* grad_out,
                                int64_t T, int64_t top_k, int64_t H, int64_t rows, moe_dtype dt,
                                void* dexpert, float* dweights, hipStream_t stream);

/*
 * moe_experts_forward_training - the experts' forward keeping a cache
 * (forward_dispatched_training). Arguments as moe_experts_forward_dispatched,
 * plus
 *   cache [rows, 3*I] dt (moe_experts_training_cache_size bytes), written:
 *         the first rows*2*I elements hold (g | u) per row, g = x W_gate^T and
 *         u = x W_up^T rounded to dt; then rows*I elements hold
 *         h = SiLU(g) * u computed from the cached g, u and rounded to dt.
 *   expert_out = h W_down^T, as the inference path.
 *   ws: moe_experts_forward_training_workspace_size(rows, E, H, I, dt).
 * x_disp, the weights and the cache must stay unchanged until
 * moe_experts_backward has run. Errors: UNSUPPORTED for dt F32 (this path
 * runs on the bf16/f16 matrix cores) and for H or 2*I above 2^22 elements.
 */
moe_status moe_experts_forward_training(const void* x_disp, const int32_t* expert_offsets,
                                        int64_t rows, int64_t E, int64_t H, int64_t I,
                                        const void* w_gate, const void* w_up, const void* w_down,
                                        moe_dtype dt, void* expert_out, void* cache, void* ws,
                                        size_t ws_bytes, hipStream_t stream);
size_t moe_experts_training_cache_size(int64_t rows, int64_t I, moe_dtype dt);
size_t moe_experts_forward_training_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                                   moe_dtype dt);

/*
 * moe_experts_backward - cache.backward(dexpert).
 *   dexpert [rows, H] dt (from moe_combine_backward), read.
 *   With dh = dexpert W_down (fp32, not rounded), s = sigmoid(g):
 *     dg = dh * u * s * (1 + g (1 - s)), du = dh * SiLU(g), both rounded to dt;
 *   dinput [rows, H] dt, written: dg W_gate + du W_up;
 *   dgate, dup [E, I, H] fp32, written: dg^T x_disp, du^T x_disp per expert;
 *   ddown [E, H, I] fp32, written: dexpert^T h per expert.
 *   An expert without rows gets zero weight gradients (also for rows = 0).
 *   ws: moe_experts_backward_workspace_size(rows, E, H, I, dt).
 */
moe_status moe_experts_backward(const void* x_disp, const int32_t* expert_offsets, int64_t rows,
                                int64_t E, int64_t H, int64_t I, const void* w_gate,
                                const void* w_up, const void* w_down, moe_dtype dt,
                                const void* cache, const void* dexpert, void* dinput,
                                float* dgate, float* dup, float* ddown, void* ws, size_t ws_bytes,
                                hipStream_t stream);
size_t moe_experts_backward_workspace_size(int64_t rows, int64_t E, int64_t H, int64_t I,
                                           moe_dtype dt);

/*
 * moe_dispatch_backward - dispatch_backward: dx[t] = sum over the slots j of
 * token t with a dispatched row of dinput[row_of_slot[t*top_k+j]], in fp32
 * in j order, stored in dt; the routing weight is not applied again (it was
 * applied in moe_combine_backward). A token without rows gets zeros.
 *   dinput [rows, H] dt (rows <= T*top_k), row_of_slot [T*top_k]: read;
 *   dx [T, H] dt: written.
 */
moe_status moe_dispatch_backward(const void* dinput, const int32_t* row_of_slot, int64_t T,
                                 int64_t top_k, int64_t H, int64_t rows, moe_dtype dt, void* dx,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
