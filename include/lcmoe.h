/*
 * lcmoe -- LongCat-Flash MoE layer with zero-computation experts, for MI355X
 * (gfx950). C ABI of liblcmoe.so.
 *
 * The layer ("LongCat-Flash", llm-wiki entity page, section 2.1
 * "Zero-Computation Experts"):
 *
 *   MoE(x_t) = sum_{i < N+Z} g_i * E_i(x_t),  E_i(x_t) = x_t for the Z
 *   zero-computation experts, a SiLU-gated FFN for the N others;
 *   the router picks K experts per token on logit + expert bias;
 *   the bias follows  db_i = mu * (K_e/K * 1/N - T_i/(K * T_all)).
 *
 * Readings where the page is silent (applied by every entry point):
 *   - the bias is added to the fp32 router logit for selection only;
 *   - gates are softmax(z) over all N+Z unbiased logits, read at the K
 *     selected experts, not renormalised;
 *   - selection order is (score descending, expert index ascending), -0 == +0;
 *   - the FFN expert is W2 (silu(W1 x) * (W3 x)) with W1 (gate) rows [0, I)
 *     and W3 (up) rows [I, 2I) stacked in one [2I][d] matrix;
 *   - the bias update changes only the N FFN experts.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to row-major contiguous arrays
 *     owned by the caller. The library keeps no device memory between calls
 *     (lcmoe_forward_noalloc's fixed array aside); scratch space is the
 *     caller's workspace `ws` of `ws_bytes` bytes (at least
 *     lcmoe_workspace_bytes(shape, T)).
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Outputs are fully overwritten. Two calls that share a workspace must
 *     be ordered (same stream). lcmoe_backward also runs part of its work on
 *     a second stream of default priority that the library creates once per
 *     device, forked from and joined back to `stream` with events inside the
 *     call; everything it enqueues is ordered before later work on `stream`.
 *   - Expert ids 0..N-1 are FFN experts, N..N+Z-1 zero-computation experts.
 *   - bf16 tensors are passed as raw 16-bit storage (`const void*`).
 *   - fp8 weights (LCMOE_W_FP8_E4M3_B128) are OCP E4M3FN codes (one byte
 *     each) with one fp32 scale per 128x128 block of each expert matrix;
 *     the weight value is fl32(code_value * scale).
 *   - Arguments are validated before anything is enqueued; on failure the
 *     status is returned and nothing runs. No C++ exception crosses the ABI
 *     and the library never aborts.
 *
 * Status codes:
 *   LCMOE_ERR_INVALID_ARG  null required pointer, T < 0, K < 1, K > N+Z,
 *                          N < 1, Z < 0, bad dtype code, mu/k_e not finite.
 *   LCMOE_ERR_UNSUPPORTED  K > 64, N+Z > 2048, d % 32 != 0, I % 32 != 0,
 *                          fp8 with d % 128 or I % 128 != 0 or d or I
 *                          above 16384, one expert's W13 of 4 GiB or
 *                          more, a tensor pointer not 16-byte aligned,
 *                          T*K >= 2^31, (forward) x of 4 GiB or more,
 *                          (backward) fp8 weights or slot rows of 4 GiB
 *                          or more (see lcmoe_backward).
 *   LCMOE_ERR_WORKSPACE    ws is NULL or ws_bytes too small.
 *   LCMOE_ERR_HIP          a HIP launch failed (hipGetLastError).
 */
#ifndef LCMOE_H
#define LCMOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCMOE_OK = 0,
  LCMOE_ERR_INVALID_ARG = 1,
  LCMOE_ERR_UNSUPPORTED = 2,
  LCMOE_ERR_WORKSPACE = 3,
  LCMOE_ERR_HIP = 4
} lcmoe_status;

typedef enum {
  LCMOE_W_BF16 = 0,          /* expert weights in bf16                         */
  LCMOE_W_FP8_E4M3_B128 = 1, /* E4M3FN codes + fp32 scale per 128x128 block    */
  /* Weights as LCMOE_W_FP8_E4M3_B128, and fp8 activations: each FFN expert's
   * input row (x_t) and intermediate row (H, after its bf16 rounding) are
   * quantized per row to E4M3FN with one fp32 scale s = fl32(amax/448)
   * (1 for a zero row), q = round-to-nearest-even of fl32(v/s), and the
   * expert GEMMs run on fp8 MFMA (fp32 accumulation, weight block scales
   * applied per 128-wide k block, the row scale after the sum). The pages
   * name FP8 quantization without its activation scheme; this is the
   * reading. Zero-computation experts still return the exact x. */
  LCMOE_W_FP8_E4M3_B128_A8 = 2
} lcmoe_wdtype;

/* Layer shape. Model table of "LongCat-Flash" (section 1): d_model 6144,
 * 512 FFN experts, 256 zero-computation experts, 12 experts per token,
 * expert intermediate size 2048. */
typedef struct {
  int32_t d_model;   /* d                                   */
  int32_t n_ffn;     /* N: FFN experts                      */
  int32_t n_zero;    /* Z: zero-computation experts         */
  int32_t top_k;     /* K: experts per token, zero included */
  int32_t d_expert;  /* I: FFN expert intermediate size     */
  int32_t w_dtype;   /* lcmoe_wdtype                        */
} lcmoe_shape;

/* Workspace bytes needed by lcmoe_route / lcmoe_permute / lcmoe_forward for
 * any T <= max_tokens. Pure host function, no HIP call. Returns 0 for an
 * invalid or unsupported shape or max_tokens < 0. Non-decreasing in
 * max_tokens. */
size_t lcmoe_workspace_bytes(const lcmoe_shape* shape, int32_t max_tokens);

/* Routing half of the layer ("LongCat-Flash" section 2.1: the router selects
 * K of the N+Z experts per token; T_i counts the tokens routed to expert i).
 *
 *   x_bf16     [T][d]   bf16 layer input (read; upcast to fp32 exactly)
 *   w_router   [E][d]   fp32 router weights, E = N+Z
 *   bias       [E]      fp32 expert bias, read for selection only
 *   topk_idx   [T][K]   int32 out: selected experts in selection order
 *   topk_gate  [T][K]   fp32 out: softmax(z_t)[topk_idx]
 *   counts     [E]      int32 out: T_i for every expert
 *   logits_out [T][E]   fp32 out, optional (NULL to skip): router logits z
 *
 * z = x W_r^T is computed with exact fp32 products (W_r is split exactly
 * into three bf16 planes, x is bf16) and fp32 accumulation. Selection uses
 * s = fl32(z + b). T == 0: counts are zeroed, nothing else is written. */
lcmoe_status lcmoe_route(const lcmoe_shape* shape, int32_t T,
                         const void* x_bf16, const float* w_router,
                         const float* bias,
                         int32_t* topk_idx, float* topk_gate,
                         int32_t* counts, float* logits_out,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Counting-sort permutation of the FFN slots of a routing (the per-expert
 * grouping that feeds the grouped expert GEMMs). Slots are the flat
 * positions j = t*K + k of topk_idx.
 *
 *   topk_idx    [T][K]  int32 in: expert ids, each in [0, E), distinct per row
 *   counts      [E]     int32 out: T_i for every expert
 *   offsets     [N+1]   int32 out: exclusive prefix sum of counts[0..N)
 *   perm        [T*K]   int32 out: entries [0, S) hold the FFN slot ids grouped
 *                       by expert, ascending inside a group (S = offsets[N]);
 *                       entries [S, T*K) are set to -1
 *   row_of_slot [T*K]   int32 out: position of slot j in perm, -1 when slot j
 *                       went to a zero-computation expert
 * Ids outside [0, E) give unspecified (but memory-safe) results. */
lcmoe_status lcmoe_permute(const lcmoe_shape* shape, int32_t T,
                           const int32_t* topk_idx,
                           int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* row_of_slot,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer ("LongCat-Flash" section 2.1, the MoE sum with
 * zero-computation experts): routing as lcmoe_route, the permutation as
 * lcmoe_permute, the SiLU-gated expert FFNs over the FFN-routed tokens only
 * (grouped GEMMs), and the weighted combine
 *   y_t = sum_k g_tk * (E_{idx_tk}(x_t) if idx_tk < N else x_t)
 * accumulated in fp32 in k order and rounded once to bf16.
 *
 *   w13        [N][2I][d]  bf16, or E4M3FN codes (fp8)
 *   w13_scale  [N][2I/128][d/128] fp32 (fp8 only; NULL for bf16)
 *   w2         [N][d][I]   bf16, or E4M3FN codes (fp8)
 *   w2_scale   [N][d/128][I/128]  fp32 (fp8 only; NULL for bf16)
 *   y_bf16     [T][d]      bf16 out
 *   topk_idx, topk_gate, counts: as lcmoe_route (written)
 *
 * Intermediate precision: expert GEMMs accumulate in fp32; the SiLU product
 * and the expert output are stored as bf16 before the next step. With fp8
 * weights each weight is rounded once, fl32(q*s) -> bf16, in registers. The
 * bias is never modified here. */
lcmoe_status lcmoe_forward(const lcmoe_shape* shape, int32_t T,
                           const void* x_bf16, const float* w_router,
                           const float* bias,
                           const void* w13, const float* w13_scale,
                           const void* w2, const float* w2_scale,
                           void* y_bf16,
                           int32_t* topk_idx, float* topk_gate, int32_t* counts,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* lcmoe_forward for fp8 weights and fp8 activations (LCMOE_W_FP8_E4M3_B128_A8)
 * that also hands the activation path's intermediates to the caller, for
 * verification harnesses: the same kernels on the same values (every output
 * of lcmoe_forward bit for bit), with the quantized token rows and the FFN
 * intermediate written to these caller buffers instead of the workspace.
 * The per-row quantization is the reading stated at LCMOE_W_FP8_E4M3_B128_A8
 * (the pages name FP8 quantization, "LongCat-Flash" section 5, without the
 * activation scheme).
 *
 *   xq  [T][d]  uint8 out: E4M3FN codes of every token row x_t
 *   xs  [T]     fp32 out: the row scales s = fl32(amax / 448)
 *   h   [S][I]  bf16 out: H = silu(x W1^T) * (x W3^T) of every FFN slot row,
 *               before its quantization
 *   hq  [S][I]  uint8 out: E4M3FN codes of H
 *   hs  [S]     fp32 out: the row scales of H
 * with S = T * min(K, N) rows allocated; row r is FFN slot row r of the
 * expert-grouped slot order (lcmoe_permute's perm: grouped by expert, slot id
 * ascending inside a group) and rows at or past the FFN slot count are not
 * written. Other arguments, errors and outputs as lcmoe_forward; also
 * UNSUPPORTED for another weight type or a buffer not 16-byte aligned, and
 * INVALID_ARG for a null buffer with T > 0. The buffers are caller-owned
 * device memory and must not overlap the workspace. */
lcmoe_status lcmoe_forward_inspect(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias,
                                   const void* w13, const float* w13_scale,
                                   const void* w2, const float* w2_scale,
                                   void* y_bf16,
                                   int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                   void* xq, float* xs, void* h, void* hq, float* hs,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the fixed device scratch array lcmoe_forward_noalloc works in. */
#define LCMOE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* lcmoe_forward for callers that cannot allocate device memory (work under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same outputs, bit for bit, with the workspace
 * taken from a fixed array of LCMOE_NOALLOC_SCRATCH_BYTES that the library
 * holds on each device it runs on (in its code object, from the first use on
 * that device until the process ends). The call allocates nothing. Arguments
 * and outputs as lcmoe_forward without ws / ws_bytes; the caller still owns
 * the inputs and outputs. A call whose workspace for its T (at most
 * lcmoe_workspace_bytes(shape, T)) exceeds the array returns
 * LCMOE_ERR_WORKSPACE before anything is enqueued; at the LongCat shape with
 * bf16 weights that admits up to about 1,000 tokens per call (decode
 * batches). Every call on one device shares that
 * device's array: two calls that can overlap on one device (other streams,
 * other host threads) race and must be ordered by the caller. The stream must
 * belong to the current device; the first call on a device looks up the
 * array's address there (LCMOE_ERR_HIP if that fails). */
lcmoe_status lcmoe_forward_noalloc(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias,
                                   const void* w13, const float* w13_scale,
                                   const void* w2, const float* w2_scale,
                                   void* y_bf16,
                                   int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                   hipStream_t stream);

/* Stages of lcmoe_forward, in launch order (for lcmoe_forward_staged). */
typedef enum {
  LCMOE_STAGE_ROUTER = 0,     /* router logits                          */
  LCMOE_STAGE_TOPK = 1,       /* biased top-K and gates                 */
  LCMOE_STAGE_PERMUTE = 2,    /* histogram, scans, stable scatter        */
  LCMOE_STAGE_GATEUP = 3,     /* grouped gate/up GEMM with the SiLU gate */
  LCMOE_STAGE_DOWN = 4,       /* grouped down GEMM                       */
  LCMOE_STAGE_COMBINE = 5,    /* weighted combine + zero-expert identity */
  LCMOE_NUM_STAGES = 6
} lcmoe_stage;

/* lcmoe_forward with stage timing for profiling harnesses: identical work,
 * plus hipEventRecord(stage_events[i], stream) before stage i and
 * stage_events[LCMOE_NUM_STAGES] after the last one (stage_events holds
 * LCMOE_NUM_STAGES + 1 caller-created events; NULL records nothing). The
 * events are recorded only once validation has passed. */
lcmoe_status lcmoe_forward_staged(const lcmoe_shape* shape, int32_t T,
                                  const void* x_bf16, const float* w_router,
                                  const float* bias,
                                  const void* w13, const float* w13_scale,
                                  const void* w2, const float* w2_scale,
                                  void* y_bf16,
                                  int32_t* topk_idx, float* topk_gate, int32_t* counts,
                                  void* ws, size_t ws_bytes, hipStream_t stream,
                                  hipEvent_t* stage_events);

/* Expert-bias update ("LongCat-Flash" section 2.1, the bias-adaptation law;
 * mu the adaptation rate, K_e the target FFN experts per token, T_i the
 * tokens routed to expert i, T_all the tokens in the global batch):
 *   for i < N:  b_i <- fl32(b_i + mu*(K_e*T_all - N*T_i) / (K*N*T_all)),
 * evaluated in fp64 in exactly that order (no contraction); b_i for i >= N
 * unchanged. One launch of N threads, ordered after routing by the stream.
 *
 *   t_all   tokens in the batch whose counts are passed (> 0)
 *   counts  [E] int32 device, read
 *   bias    [E] fp32 device, updated in place */
lcmoe_status lcmoe_bias_update(const lcmoe_shape* shape, int32_t t_all,
                               const int32_t* counts, double mu, double k_e,
                               float* bias, hipStream_t stream);

/* Backward of the layer ("LongCat-Flash" section 2.1: y_t = sum over the K
 * selected of the N+Z experts of g_i E_i(x_t), g from one softmax over all
 * experts, a zero expert the identity): the gradients of <dy, y> with respect
 * to x, W_r and the expert weights. The selection is piecewise constant and
 * the expert bias enters it only, so neither has a gradient. Chain rule:
 *   dg_tk = <dy_t, v_tk>;  FFN slot: dh = g W2^T dy_t, du = [dh c silu'(a);
 *   dh silu(a)] (u = W13 x_t = [a; c]), dW2 += g dy_t h^T, dW13 += du x_t^T,
 *   dx_t += W13^T du;  zero slot: dx_t += g dy_t;
 *   dz_t = p_t (dp_t - <dp_t, p_t>) with dp_t[idx_tk] = dg_tk;
 *   dW_r = dz^T x;  dx_t += W_r^T dz_t.
 * The routing and the expert pre-activations u are recomputed from x (the
 * same kernels as the forward, so the same selection). bf16 weights only.
 * Expert GEMMs: bf16 operands (u and W2^T dy kept in fp32, du and g h
 * rounded to bf16), fp32 accumulation; router gradients at fp32 accuracy
 * (bf16 MFMA on exact three-plane splits of dz and W_r, fp32 accumulation).
 *
 *   x_bf16, w_router, bias, w13, w2   as for lcmoe_forward (read)
 *   dy_bf16    [T][d] bf16 device, read: gradient of the loss w.r.t. y
 *   dx         [T][d] fp32 device, written
 *   dw_router  [E][d] fp32 device, written
 *   dw13       [N][2I][d] bf16 device, written (zero for untouched experts)
 *   dw2        [N][d][I] bf16 device, written (zero for untouched experts)
 *   ws         >= lcmoe_backward_workspace_bytes(shape, T) bytes
 * Errors as lcmoe_forward; UNSUPPORTED for fp8 weights and for
 * T * max(d, 2I) * 2 >= 2^32 (the grouped GEMMs address an expert's slot
 * rows with 32-bit byte offsets). T = 0 zeroes the weight gradients.
 * The weight-gradient GEMMs (dW2, dW13; HBM writes) run on the library's
 * second stream, on part of the CUs, beside dx and the router gradients
 * (HBM reads) on `stream`; the call joins them back before returning, so
 * the outputs are ordered on `stream` like any other work. The first call
 * on a device creates that stream and its two events (LCMOE_ERR_HIP if that
 * fails), so under HIP graph capture make one call before capturing; the
 * fork and join are then captured like the kernels. The staged variant runs
 * every stage in order on `stream` (same kernels, same bits). */
size_t lcmoe_backward_workspace_bytes(const lcmoe_shape* shape, int32_t max_tokens);
lcmoe_status lcmoe_backward(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                            const float* w_router, const float* bias, const void* w13,
                            const void* w2, const void* dy_bf16, float* dx, float* dw_router,
                            void* dw13, void* dw2, void* ws, size_t ws_bytes,
                            hipStream_t stream);
/* The same call, recording the caller's 10 events (array, may be NULL) at
 * stage boundaries: start, routing (with the gather of each FFN slot's x
 * and dy rows into slot order), W2^T dy, u with the SiLU backward, dg and
 * the router's dz, dx rows, dW2, dW13, router gradients, dx. */
lcmoe_status lcmoe_backward_staged(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                   const float* w_router, const float* bias, const void* w13,
                                   const void* w2, const void* dy_bf16, float* dx,
                                   float* dw_router, void* dw13, void* dw2, void* ws,
                                   size_t ws_bytes, hipStream_t stream, hipEvent_t* stage_events);

/* Training pair. lcmoe_forward_train is lcmoe_forward (bf16 weights) that
 * also stores, for every FFN slot row, the expert pre-activations
 * u = [W1 x; W3 x] in fp32, the accumulators its gate/up epilogue holds
 * before the SiLU gate. lcmoe_backward_saved is lcmoe_backward taking those
 * rows instead of recomputing u = W13 x, which saves one read of every
 * touched expert's W13 for one write and one read of u. The routing is
 * recomputed (same kernels, so the same selection and slot order): the
 * backward must see the same x, router weights and bias as the forward that
 * saved u.
 *
 *   u_save, u_saved  [T*min(K,N)][2I] fp32 device, written by the forward,
 *                    read by the backward: row r is FFN slot row r of the
 *                    layer's expert-grouped slot order (rows past the slot
 *                    count are not touched)
 * Other arguments as lcmoe_forward / lcmoe_backward (no fp8 scales: bf16
 * weights only). Errors as those calls; UNSUPPORTED for fp8 weights or a
 * misaligned u buffer, INVALID_ARG for a null u buffer with T > 0. */
lcmoe_status lcmoe_forward_train(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                 const float* w_router, const float* bias, const void* w13,
                                 const void* w2, void* y_bf16, int32_t* topk_idx,
                                 float* topk_gate, int32_t* counts, void* u_save, void* ws,
                                 size_t ws_bytes, hipStream_t stream);
lcmoe_status lcmoe_backward_saved(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                  const float* w_router, const float* bias, const void* w13,
                                  const void* w2, const void* dy_bf16, const void* u_saved,
                                  float* dx, float* dw_router, void* dw13, void* dw2, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Router-side statistics ("LongCat-Flash" section 2.1, load-balance control:
 * the device-level load-balance loss L_LB = alpha * sum_{j=1..D+1} f_j P_j
 * with the zero-computation experts as group D+1; the training-stability
 * section, activation stability: the hidden z-loss
 * L_Z = lambda/T * sum_t (log sum_i exp|h_t^i|)^2). Forward values only; no
 * gradients. Definitions where the page is silent:
 *   groups  FFN expert i is in group i / (N/D) (D consecutive blocks, the
 *           placement of expert parallelism over D devices); every zero
 *           expert is in group D+1.
 *   P_j     mean over the T tokens of the softmax mass of group j, softmax
 *           over all N+Z unbiased logits.
 *   f_j     group j's share of the T*K selected slots (from counts) divided
 *           by its target share: K_e/(K*D) for each FFN group, (K-K_e)/K for
 *           the zero group (K_e = K sets no zero-group target: f = 0). Routing
 *           at the target ratio K_e : (K-K_e), even over the FFN groups,
 *           gives f_j = 1 for every group.
 *   h_t     the layer input x_t (i runs over d_model).
 * Deterministic: fixed summation orders (per-token values in fp32, sums over
 * tokens and groups in fp64), no atomics. T = 0 writes zeros.
 *
 *   x_bf16    [T][d] bf16 device, read
 *   logits    [T][E] fp32 device, read (the router logits lcmoe_route
 *             exports through logits_out)
 *   counts    [E] int32 device, read (tokens per expert of the same routing)
 *   n_groups  D >= 1, divides N
 *   k_e       target FFN experts per token, 0 < k_e <= K
 *   alpha, lambda  finite coefficients
 *   stats     [2 + 2(D+1)] fp64 device, written: L_LB, L_Z, f_1..f_{D+1},
 *             P_1..P_{D+1}
 *   ws        >= lcmoe_router_stats_workspace_bytes(shape, n_groups) bytes
 * Errors: INVALID_ARG (null pointer, T < 0, bad n_groups, k_e or
 * coefficients), UNSUPPORTED (bad shape, misaligned x or logits), WORKSPACE,
 * ERR_HIP. */
size_t lcmoe_router_stats_workspace_bytes(const lcmoe_shape* shape, int32_t n_groups);
lcmoe_status lcmoe_router_stats(const lcmoe_shape* shape, int32_t T, const void* x_bf16,
                                const float* logits, const int32_t* counts, int32_t n_groups,
                                double k_e, double alpha, double lambda, double* stats,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Static string naming a status code. */
const char* lcmoe_status_str(lcmoe_status status);

#ifdef __cplusplus
}
#endif

#endif /* LCMOE_H */
