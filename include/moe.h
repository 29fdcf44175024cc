/*
 * moe.h -- C ABI of the sparse-MoE layer forward on one MI355X (gfx950).
 *
 * The forward is split at the semantic boundaries that the RL-Kernel roadmap
 * ("DSV4 Flash MoE Train-Inference Consistency Roadmap", Problem 2:
 * Single-Operator Boundaries May Not Be Meaningful) asks to compare:
 *   routing   -> moe_route    router logits, top-k ids, top-k weights
 *   dispatch  -> moe_permute  per-expert counts, offsets, token permutation
 *   expert    -> moe_experts  SwiGLU expert MLPs as one grouped GEMM pair
 *   reduction -> moe_combine  weighted combine in a fixed order and dtype
 * and moe_forward runs all of them (plus the shared expert) on one stream.
 *
 * Conventions common to every entry point
 *   - Pointers named as device data are HIP device pointers; the caller owns
 *     every buffer.  The library allocates nothing, keeps no pointer after it
 *     returns, never synchronises the stream and holds no state between calls
 *     (the selection bias is an input, never state: SpecForge pull request
 *     #1003, review thread, the router forward is stateless).
 *   - Tensors are row-major and contiguous.  bf16 tensors hold IEEE bfloat16
 *     bit patterns.  "Operand dtype" is moe_shape.dtype: MOE_BF16 means bf16
 *     activations and weights with fp32 accumulation; MOE_F32 means fp32
 *     activations and weights.
 *   - Arguments are validated before anything is launched.  On any error no
 *     kernel runs, outputs are untouched and the status says why; the text of
 *     the last error of the calling thread is in moe_last_error().  There is
 *     no fallback to other numerics (fail closed: RL-Kernel roadmap, issue
 *     buckets).  T == 0 returns MOE_OK and launches nothing (moe_backward
 *     then zeroes the weight gradients: sums over no tokens); buffers of T
 *     rows (x, out, dout, dx, the trace) and the workspace may then be NULL.
 *   - Alignment: activations, weights, outputs, gradients, y, shared_out and
 *     the workspace are moved in 16-byte vectors and must start on a 16-byte
 *     boundary; the int32 arrays, the per-token float32 arrays, logits and
 *     sel_bias on a 4-byte one.  Any other pointer is MOE_ERR_INVALID.
 *   - Kernel faults surface at the caller's next synchronisation; launch
 *     errors return MOE_ERR_HIP.
 *   - Supported shapes: D, I (and Is when non-zero) multiples of 64;
 *     1 <= E <= 1024; 1 <= K <= min(E, 16); T*K < 2^31; device gfx950.
 *     Anything else returns MOE_ERR_UNSUPPORTED (or MOE_ERR_INVALID for
 *     values that cannot describe a layer at all).
 *   - Inputs must be finite; NaN or Inf inputs give unspecified outputs.
 *   - Results are deterministic and batch invariant: a token's ids, weights
 *     and output bits do not depend on T, on the other tokens, on padding or
 *     on token order.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,      /* a NULL required pointer, a negative size, an unknown enum */
    MOE_ERR_UNSUPPORTED = 2,  /* a valid layer this library does not run (shape limits, device) */
    MOE_ERR_WORKSPACE = 3,    /* ws is NULL or ws_bytes below moe_workspace_size() */
    MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* Router score function (RL-Kernel roadmap, Problem 1: router softmax; SpecForge
 * pull request #1003 commit notes: sigmoid and sqrtsoftplus routers).  The
 * score is computed in float64 from float64-accumulated logits.
 * MOE_SQRTSOFTPLUS is read as sqrt(log(1 + e^l)) (the pages name it without a
 * formula). */
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1, MOE_SQRTSOFTPLUS = 2 } moe_score;

/* Combine arithmetic (moe_combine, moe_forward).
 *   MOE_COMBINE_F32_FOLD: float32 left fold in ascending expert id (the
 *     default; 6 routed terms give 6!/2 = 360 distinct orders, the count of
 *     arXiv 2607.28097, Abstract).
 *   MOE_COMBINE_F64: the products w * y are exact in float64 and summed there
 *     in ascending expert id, the shared term added, then rounded once to the
 *     output dtype.  Whenever that float64 sum is exact (the products'
 *     exponents span less than about 20 bits) the result does not depend on
 *     the order of the terms: an order-invariant reduction. */
typedef enum { MOE_COMBINE_F32_FOLD = 0, MOE_COMBINE_F64 = 1 } moe_combine_mode;

/* The layer's profile (the ModelProfile of the RL-Kernel roadmap, WS1). */
typedef struct {
    int64_t T;          /* tokens in this call */
    int32_t D;          /* hidden size */
    int32_t E;          /* routed experts */
    int32_t K;          /* experts per token */
    int32_t I;          /* routed expert SwiGLU intermediate size */
    int32_t Is;         /* shared expert intermediate size, 0 = no shared expert */
    int32_t score;      /* moe_score */
    int32_t renorm;     /* 1: weights renormalised over the K selected experts */
    float route_scale;  /* multiplies the (renormalised) weights; finite, > 0 */
    int32_t dtype;      /* moe_dtype: operand dtype of x, weights, expert activations and outputs */
    int32_t combine;    /* moe_combine_mode */
    /* Group-limited select (SpecForge pull request #1003 commit notes on select:
     * DeepSeek-V3's group-limited routing, named without a formula; read as:
     * experts form n_group groups of E/n_group consecutive ids, a group's
     * score is the sum of its two largest choices, the topk_group best groups
     * are kept, ties to the lower group id, and the K experts are chosen
     * among the kept groups).  n_group 0 or 1: no grouping.  Otherwise E must
     * be a multiple of n_group with at least 2 experts per group, n_group
     * <= 64, 1 <= topk_group <= n_group and K <= topk_group * E / n_group. */
    int32_t n_group;
    int32_t topk_group;
} moe_shape;

/* Weights of one layer (device pointers, operand dtype unless noted).
 *   router          [E, D]
 *   gate_up         [E, 2I, D]  rows 0..I-1 gate projection, rows I..2I-1 up projection
 *   down            [E, D, I]
 *   gate_up_shared  [2Is, D]    (NULL when Is == 0)
 *   down_shared     [D, Is]     (NULL when Is == 0)                                  */
typedef struct {
    const void* router;
    const void* gate_up;
    const void* down;
    const void* gate_up_shared;
    const void* down_shared;
} moe_weights;

/* Optional copies of every boundary tensor of moe_forward (the SemanticTrace of
 * the RL-Kernel roadmap, WS1).  Each pointer may be NULL; a non-NULL pointer
 * must hold the full tensor and receives exactly what the corresponding stage
 * entry point would write.
 *   logits      float [T, E]      router logits (float64 accumulation rounded to float32)
 *   topk_ids    int32 [T, K]
 *   topk_w      float [T, K]
 *   counts      int32 [E]
 *   offsets     int32 [E+1]
 *   perm_token  int32 [T*K]       first offsets[E] entries written
 *   inv_pos     int32 [T, K]
 *   y           operand dtype [T*K, D]   routed expert outputs, permuted order
 *   shared_out  operand dtype [T, D]     shared expert output (Is > 0)            */
typedef struct {
    float* logits;
    int32_t* topk_ids;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm_token;
    int32_t* inv_pos;
    void* y;
    void* shared_out;
} moe_trace;

/* Workspace bytes moe_forward needs for this shape.  The same amount is enough
 * for every stage entry point.  Host-only; launches nothing. */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* Routing (RL-Kernel roadmap, Problem 1 and the routing boundary of Problem 2;
 * SpecForge pull request #1003, commit notes on the router).
 *   logits[t,e] = sum_d x[t,d] * router[e,d], accumulated in float64 from
 *   float32 partial sums of 256 products each (bf16 mode) or in float64 (f32 mode);
 *   s = softmax over e, sigmoid or sqrtsoftplus, in float64;
 *   choice = s + sel_bias[e] (sel_bias may be NULL);
 *   the K experts with the largest choice are selected, ties to the lower id;
 *   topk_ids[t,:] lists them in ascending id order;
 *   topk_w[t,j] = s[id_j] (unbiased), divided by the sum over the selection when
 *   renorm, times route_scale, rounded once to float32.
 * x [T,D] and router [E,D] in operand dtype; sel_bias float [E] or NULL;
 * mask uint8 [T] or NULL (0 = masked token: ids -1, weights 0);
 * logits float [T,E] or NULL (optional export); topk_ids int32 [T,K];
 * topk_w float [T,K]; ws of at least moe_workspace_size() bytes. */
moe_status moe_route(const moe_shape* shape, const void* x, const void* router,
                     const float* sel_bias, const uint8_t* mask, float* logits,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Dispatch (RL-Kernel roadmap, Problem 2: token-to-expert map, valid token
 * counts, padding provenance).  A stable counting sort of the T*K (token, slot)
 * pairs by expert id, built without atomics.
 *   counts[e]        pairs routed to e (slots holding -1 are skipped)
 *   offsets[e]       exclusive prefix sum of counts, offsets[E] = kept pairs
 *   perm_token[p]    token of row p of the expert-sorted order; within one
 *                    expert the tokens ascend
 *   inv_pos[t,j]     row of pair (t,j) in that order, -1 for skipped slots
 * topk_ids int32 [T,K]: ids in [0,E), or -1 for a slot without an expert; a
 * slot holding any other value (< -1 or >= E) is skipped like -1.  A token
 * is expected to list distinct ids (tokens then ascend within an expert);
 * the kernels do not check it.  Outputs as above (device). */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv_pos,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert MLPs (RL-Kernel roadmap, Problem 2: gate_and_up -> down; SpecForge
 * pull request #1003, "Design notes": the routed experts as grouped GEMMs).
 * For every group g in [0, shape->E) and row p in [offsets[g], offsets[g+1]):
 *   h = x[src(p)] . gate_up[g]^T            (fp32 accumulate, K order fixed)
 *   a = silu(h[0:I]) * h[I:2I]              (fp32; rounded to bf16 in bf16 mode)
 *   y[p] = a . down[g]^T                    (fp32 accumulate; bf16 in bf16 mode)
 * src(p) = perm_token[p], or p when perm_token is NULL.  offsets int32 [E+1]
 * (device), or NULL for one group of all T rows (requires E == 1).  The row
 * count is at most T*K.  gate_up [E,2I,D], down [E,D,I], x [*,D], y [T*K,D],
 * all operand dtype.  The shared expert is this call with E = K = 1, I = Is,
 * perm_token = offsets = NULL. */
moe_status moe_experts(const moe_shape* shape, const void* x, const int32_t* perm_token,
                       const int32_t* offsets, const void* gate_up, const void* down,
                       void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Weighted combine, the final reduction (RL-Kernel roadmap, Problem 3; arXiv
 * 2607.28097, Abstract: operand conversion, accumulator precision and
 * reduction order belong to the numerical contract).  For each kept token t:
 *   acc = +0.0f
 *   for j = 0..K-1 (ascending expert id):  acc = fl32(acc + fl32(topk_w[t,j] * f32(y[inv_pos[t,j]])))
 *   if shared_out:                         acc = fl32(acc + f32(shared_out[t]))
 *   out[t] = acc rounded to bf16 nearest-even (out_dtype MOE_BF16) or acc (MOE_F32)
 * No fused multiply-add.  With shape->combine == MOE_COMBINE_F64 the same
 * terms are formed and summed in float64 and the sum is rounded once (to bf16
 * or float32, nearest-even).  A slot whose inv_pos is -1 contributes nothing
 * (its weight is not read); a token whose inv_pos slots are all -1 gets a +0
 * row.  inv_pos entries other than -1 must be rows of y.
 * y [T*K,D] and shared_out [T,D] (or NULL) in operand dtype; inv_pos int32
 * [T,K]; topk_w float [T,K]; out [T,D] in out_dtype. */
moe_status moe_combine(const moe_shape* shape, const void* y, const int32_t* inv_pos,
                       const float* topk_w, const void* shared_out, int32_t out_dtype,
                       void* out, hipStream_t stream);

/* The whole layer: route, permute, routed experts, shared expert (when Is > 0,
 * ungated, on every token: SpecForge pull request #1003, "Design notes"), and
 * combine, in that order on one stream.  out [T,D] in out_dtype; trace may be
 * NULL.  Bitwise equal to calling the stages one after another. */
moe_status moe_forward(const moe_shape* shape, const moe_weights* weights, const void* x,
                       const float* sel_bias, const uint8_t* mask, int32_t out_dtype,
                       void* out, const moe_trace* trace, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Bytes of the fixed device scratch of moe_forward_noalloc (64 MiB per device). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts that
 * forbid allocation during the forward).  It runs exactly the kernels of
 * moe_forward, with the same results bit for bit, on a scratch array that the
 * library holds in device memory: MOE_NOALLOC_SCRATCH_BYTES per device, set
 * aside when the library's device code is loaded on that device and kept
 * until the process ends.  The call allocates nothing and frees nothing.
 * Shapes whose moe_workspace_size() exceeds MOE_NOALLOC_SCRATCH_BYTES return
 * MOE_ERR_UNSUPPORTED before anything runs (at 64 MiB: decode and moderate
 * prefill batches, e.g. up to 796 tokens of a 4096-wide, 256-expert, top-6
 * layer with a 2048-wide routed and shared expert).  Every call on one device uses the same
 * scratch, which keeps what the last call left there; the forward needs no
 * zeroed memory (it issues no memset), and no value left by an earlier call
 * reaches an output, exactly as for moe_forward's workspace.  Calls that
 * overlap on one device (two streams, or two host threads, without ordering
 * between them) race on the scratch and give undefined results.  Arguments
 * otherwise as in moe_forward. */
moe_status moe_forward_noalloc(const moe_shape* shape, const moe_weights* weights, const void* x,
                               const float* sel_bias, const uint8_t* mask, int32_t out_dtype, void* out,
                               const moe_trace* trace, hipStream_t stream);

/* Routing replay (RL-Kernel roadmap, "R3 Should Not Be A Prerequisite": the
 * experts a token used in another run are replayed, the router still scores
 * them).  The router logits and scores are computed as in moe_route, but the
 * K experts of token t are replay_ids[t*K .. t*K+K-1] (int32 [T,K], device)
 * instead of the K largest choices; the weights are this router's scores of
 * those experts, renormalised and scaled as in moe_route, and topk_ids
 * returns the replayed ids in ascending order with their weights.  A token
 * that is masked, or whose replayed ids are not K distinct ids in [0, E)
 * (for instance -1 rows of a masked token), is treated as masked.  No
 * selection bias takes part.  Outputs and workspace as in moe_route. */
moe_status moe_route_replay(const moe_shape* shape, const void* x, const void* router, const int32_t* replay_ids,
                            const uint8_t* mask, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* moe_forward with moe_route_replay in place of moe_route (replay_ids as
 * there).  Everything after routing, and the trace, as in moe_forward. */
moe_status moe_forward_replay(const moe_shape* shape, const moe_weights* weights, const void* x,
                              const int32_t* replay_ids, const uint8_t* mask, int32_t out_dtype, void* out,
                              const moe_trace* trace, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gradients of one layer (device pointers, float32, row-major; the shared
 * ones are used only when Is > 0).
 *   dx               [T, D]
 *   d_router         [E, D]
 *   d_gate_up        [E, 2I, D]
 *   d_down           [E, D, I]
 *   d_gate_up_shared [2Is, D]
 *   d_down_shared    [D, Is] */
typedef struct {
    float* dx;
    float* d_router;
    float* d_gate_up;
    float* d_down;
    float* d_gate_up_shared;
    float* d_down_shared;
} moe_grads;

/* Workspace bytes moe_backward needs for this shape (host-only). */
moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes);

/* Backward of the layer (RL-Kernel roadmap: the scope list names forward +
 * backward with a deterministic reduction order; the issue-bucket table asks
 * for a single-GPU forward + backward).  Read as the gradients of moe_forward
 * with the top-k selection fixed (the selection bias gets none) and the bf16
 * rounding points passed straight through, given dout = dL/d(out) [T, D] in
 * the operand dtype:
 *   dY_p = bf16(w_j dout_t); dw_j = <dout_t, y_p> (float64);
 *   per expert (gate_up rows H recomputed in float32):
 *     dA = dY W2_e; dH = [dA u silu'(g), dA silu(g)] (bf16);
 *     dW2_e = dY_e^T A_e (A: the forward's bf16 activation); dX_e = dH W1_e;
 *     dW1_e = dH_e^T X_e;
 *   the shared expert likewise with dY = dout on kept tokens;
 *   router: the weights' gradient through renormalisation and route_scale,
 *     then through the score function, to dl [T, E] (bf16 operand);
 *     dx += dl W_r; d_router = dl^T x;
 *   dx_t = sum of the token's routed dX rows in ascending expert id, then the
 *     shared and the router terms, in float32; masked tokens get dx = 0.
 * bf16 operands only, and 2*T*K*max(D, 2I) and 2*T*max(D, 2Is) below
 * 4 GiB (MOE_ERR_UNSUPPORTED otherwise); float32 accumulation.  Every reduction has a fixed order and no atomics: repeated calls give the
 * same bits, and dx of a token does not depend on the other tokens.
 * fwd: the trace of the moe_forward call being differentiated, with
 * topk_ids, topk_w, offsets, perm_token, inv_pos and y set (the other fields
 * are not read).  Every pointer of grads is written in full (experts no token
 * picked get zero gradients; with T == 0 every weight gradient is zero and
 * ws may be NULL).  ws: moe_backward_workspace_size() bytes. */
moe_status moe_backward(const moe_shape* shape, const moe_weights* weights, const void* x, const uint8_t* mask,
                        const moe_trace* fwd, const void* dout, const moe_grads* grads, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Text of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
