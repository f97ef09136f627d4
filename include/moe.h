/*
 * moe.h - C ABI of a sparse Mixture-of-Experts FFN layer forward with
 * token-choice top-k routing, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the pages describe as Gate -> Dispatch -> Expert
 * -> Combine ("Top-k 路由" page, figure "Top-k 路由的完整生命週期"; the
 * "别只比较 Top-k" page, steps Score / Select / Merge / Execute), with the
 * Tiny-MoE walk-through ("从 Dense FFN 到 MoE", sections 3-8) fixing the
 * tensor shapes: tokens are the rows of x [T, D], experts are bias-free
 * nn.Linear stacks, the combine accumulates (index_add).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers unless stated otherwise, owned
 *     by the caller, 16-byte aligned, dense row-major, and valid until the
 *     work enqueued on `stream` has completed.  Inputs are never written.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream: no host synchronisation,
 *     no device-to-host reads, no device allocation or free.  (The layer
 *     forward also forks work onto a library-owned stream and joins it back;
 *     see moe_layer_forward.)
 *   - Validation is synchronous and happens before anything is enqueued: when
 *     a call returns anything but MOE_OK, nothing was launched.  A launch
 *     failure returns MOE_ERR_HIP (the HIP error is cleared and its text is
 *     available from moe_last_error()).  Faults inside kernels surface at the
 *     caller's next synchronisation, as for any HIP work.
 *   - The library keeps no global mutable state besides a thread-local error
 *     string; calls are re-entrant.  Two calls that share an output or a
 *     workspace buffer must be ordered by the caller (same stream).
 *   - Results are deterministic: the same inputs give bitwise the same
 *     outputs (no order-dependent floating-point atomics).
 *   - Element types: MOE_F32 = IEEE float32, MOE_BF16 = bfloat16 (uint16
 *     storage).  act_dtype is the type of x, expert weights, y and the
 *     intermediates; router_dtype the type of the router weight.
 *     Supported pairs: (F32, F32), (BF16, F32), (BF16, BF16).
 *   - Size limits: 1 <= E <= 1024, 1 <= k <= min(E, 32), D and F multiples of
 *     8 (of 4 for MOE_F32 activations), T >= 0.  Outside: MOE_ERR_UNSUPPORTED
 *     (or MOE_ERR_INVALID_ARGUMENT for values that are meaningless).
 *   - Operand spans: the kernels address each matrix operand with 32-bit
 *     byte offsets, so every one of them must span at most 0xFFE00000 bytes
 *     (4 GiB - 2 MiB): x [T, D]; the permuted rows [A_cap, D] and the
 *     activations [A_cap, F]; one expert's w13 [n_mat F, D] and w2 [D, F];
 *     the router weight as [E, 3 D] float32; the shared experts' [T, S F_s],
 *     [2 S F_s, D] and [D, S F_s]; for the backward also [A_cap, n_mat F]
 *     and [T, 2 S F_s] bfloat16.  A configuration past any of them is
 *     rejected with MOE_ERR_UNSUPPORTED by every call that takes it
 *     (moe_capacity and moe_workspace_size included), before any launch.
 *     Example: at D = 7168, k = 8 (bf16, dropless) T may be at most 37,430.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null required pointer, bad size, misalignment */
  MOE_ERR_UNSUPPORTED = 2,        /* valid but not implemented combination */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4,                /* a HIP launch or API call failed */
  MOE_ERR_DEBUG_CHECK = 5         /* MOE_DEBUG=1: a table failed its host-side check */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Scoring rule ("Top-k 路由" page, 門控函式的數學形式 Step 2 and its note;
 * "别只比较 Top-k" page, Score and Merge steps):
 *   MOE_SOFTMAX_TOPK : p = softmax(s) over all E experts, top-k on p; weight
 *                      p_sel, divided by sum p_sel when renormalize != 0
 *                      (renormalize = 0 is Switch's raw top-1 probability).
 *   MOE_TOPK_SOFTMAX : top-k on s, weight = softmax over the k selected logits.
 *   MOE_SIGMOID_BIAS : a = sigmoid(s); top-k on a + b (b = per-expert selection
 *                      bias, selection only); weight a_sel / sum a_sel
 *                      (a_sel when renormalize = 0).
 * Ties are broken toward the lower expert index; slots are in descending
 * score order. */
typedef enum { MOE_SOFTMAX_TOPK = 0, MOE_TOPK_SOFTMAX = 1, MOE_SIGMOID_BIAS = 2 } moe_scoring;

/* Expert FFN ("从 Dense FFN 到 MoE" §3): SwiGLU down(silu(gate x) * up x), or
 * the classic W_out gelu(W_in x) with the exact erf GELU.  No biases. */
typedef enum { MOE_SWIGLU = 0, MOE_GELU = 1 } moe_activation;

typedef struct {
  int32_t num_tokens;      /* T */
  int32_t d_model;         /* D */
  int32_t num_experts;     /* E: routed experts */
  int32_t top_k;           /* k */
  int32_t d_ff;            /* F: routed expert intermediate size */
  int32_t num_shared;      /* S: always-on shared experts (0 = none; SwiGLU only) */
  int32_t d_ff_shared;     /* F_s: intermediate size of one shared expert */
  int32_t scoring;         /* moe_scoring */
  int32_t renormalize;     /* used by MOE_SOFTMAX_TOPK and MOE_SIGMOID_BIAS */
  int32_t activation;      /* moe_activation of the routed experts */
  int32_t act_dtype;       /* moe_dtype of x, expert weights, y, intermediates */
  int32_t router_dtype;    /* moe_dtype of the router weight */
  float capacity_factor;   /* <= 0: dropless.  Otherwise per-expert capacity
                              C = ceil(CF * T * k / E), evaluated in double
                              precision from this float value ("Top-k 路由"
                              容量因子 section).  Assignments beyond the first C
                              of an expert, in token order, are dropped. */
} moe_config;

/* Capacity C (INT32_MAX when dropless) and the row bound A_cap of the permuted
 * buffers: A_cap = T*k when dropless, else min(T*k, E*C).  Host pointers. */
moe_status moe_capacity(const moe_config* cfg, int32_t* capacity, int32_t* rows_cap);

typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_EXPERT_FFN = 2,      /* routed experts: max_rows = A_cap, d_ff = F */
  MOE_OP_SHARED_FFN = 3,      /* shared experts: max_rows = T, d_ff = S*F_s */
  MOE_OP_LOAD_STATS = 4,
  MOE_OP_LAYER = 5,
  MOE_OP_EXPERT_CHOICE = 6,   /* moe_expert_choice_forward */
  MOE_OP_LAYER_BACKWARD = 7   /* moe_layer_backward */
} moe_op;

/* Workspace bytes that entry point `op` needs for `cfg` (host output).  A
 * workspace is caller-owned device memory, 256-byte aligned; its contents on
 * entry do not matter and on exit are unspecified. */
moe_status moe_workspace_size(const moe_config* cfg, int32_t op, size_t* bytes);

/* Gate: router logits s = W_g x ("Top-k 路由" Step 1; "从 Dense FFN 到 MoE"
 * §4 Router), scoring, top-k selection and weights (Step 2 and its note;
 * the glossary's TopKRouter; the "别只比较 Top-k" Select and Merge steps).
 *   x        [T, D]  act_dtype
 *   w_router [E, D]  router_dtype (nn.Linear weight layout [out, in])
 *   sel_bias [E]     float32, MOE_SIGMOID_BIAS only (NULL = zero bias)
 *   topk_idx [T, k]  int32 out: expert ids, slot 0 = best
 *   topk_w   [T, k]  float32 out: combine weights
 *   probs    [T, E]  float32 out or NULL: per-token soft probabilities used
 *                    by the balance loss (softmax p; a / sum a for sigmoid)
 *   ws       workspace of moe_workspace_size(MOE_OP_ROUTE) bytes
 * Selection is taken in double precision wherever the single-precision
 * scores of a token are too close to decide it (near-tie refinement), so the
 * chosen experts are those of the exact logits except at exact ties. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* sel_bias, int32_t* topk_idx, float* topk_w,
                     float* probs, void* ws, size_t ws_bytes, void* stream);

/* Dispatch ("从 Dense FFN 到 MoE" §5: per-expert (token, slot) lists in
 * row-major order; capacity and overflow per "Top-k 路由" 容量因子 and the
 * "别只比较 Top-k" mechanism table).
 *   topk_idx     [T, k]     int32 in
 *   x            [T, D]     act_dtype in, or NULL (indices only)
 *   counts       [E]        int32 out: assignments per expert before capacity
 *   offsets      [E+1]      int32 out: exclusive scan of kept counts;
 *                           offsets[E] = kept rows A
 *   row_of       [T, k]     int32 out: permuted row of (t, j), -1 = dropped
 *   token_of_row [A_cap]    int32 out: source token of each row; entries from
 *                           offsets[E] on are set to -1
 *   x_perm       [A_cap, D] act_dtype out, or NULL: x_perm[r] = x[token_of_row[r]]
 *                           for r < offsets[E]; later rows are not written
 * Rows are grouped by ascending expert id and, inside an expert, by ascending
 * token.  Bit-exact and deterministic.  Ids outside [0, E) and repeats of an
 * id already used by an earlier slot of the same token (neither is produced by
 * moe_route) are skipped: their row_of is -1 and they are not counted. */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* row_of,
                       int32_t* token_of_row, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* Grouped expert FFN ("从 Dense FFN 到 MoE" §3 expert, §5 expert batches; the
 * "别只比较 Top-k" Execute step: grouped GEMM).  Group g owns rows
 * [offsets[g], offsets[g+1]) and applies expert g:
 *   SwiGLU: y = (silu(X Wg^T) * (X Wu^T)) Wd^T,  GELU: y = gelu(X Win^T) Wout^T
 *   num_groups  G >= 1
 *   d_ff        F of these experts
 *   activation  moe_activation (MOE_GELU not allowed for shared experts)
 *   max_rows    row bound of x rows / y rows (host value)
 *   x_in        act_dtype: [max_rows, D], or [*, D] when gather_rows is given
 *   gather_rows [max_rows] int32 or NULL: row r reads x_in[gather_rows[r]]
 *   offsets     [G+1] int32 device, non-decreasing, offsets[G] <= max_rows;
 *               NULL means one group of max_rows rows
 *   w13         [G, 2F, D] (SwiGLU: gate rows 0..F-1, up rows F..2F-1) or
 *               [G, F, D] (GELU), act_dtype
 *   w2          [G, D, F] act_dtype
 *   y_out       [max_rows, D] act_dtype out (rows from offsets[G] on untouched)
 *   ws          workspace: moe_workspace_size(MOE_OP_EXPERT_FFN) for the
 *               routed call, (MOE_OP_SHARED_FFN) for the shared call; in
 *               general max_rows * F elements of act_dtype, 256-byte rounded.
 * Shared experts (S SwiGLU experts, weight 1, every token; "别只比较 Top-k"
 * six-family table) are one call with G = 1, F = S*F_s, offsets = NULL and the
 * concatenated layout w13 = [gate_0..gate_{S-1}; up_0..up_{S-1}] [2SF_s, D],
 * w2 = [down_0 | ... | down_{S-1}] [D, S F_s]. */
moe_status moe_expert_ffn(const moe_config* cfg, int32_t num_groups, int32_t d_ff,
                          int32_t activation, int32_t max_rows, const void* x_in,
                          const int32_t* gather_rows, const int32_t* offsets,
                          const void* w13, const void* w2, void* y_out,
                          void* ws, size_t ws_bytes, void* stream);

/* Combine ("从 Dense FFN 到 MoE" §6 index_add; "Top-k 路由" Step 3):
 *   y[t] = sum_{j : row_of[t,j] >= 0} topk_w[t,j] * y_perm[row_of[t,j]] + y_shared[t]
 *   y_perm   [A_cap, D] act_dtype, row_of [T, k], topk_w [T, k] float32
 *   y_shared [T, D] act_dtype or NULL; y [T, D] act_dtype out.
 * y may alias y_shared (in-place accumulate); no other aliasing.  Sums are
 * accumulated in float32 in slot order.  A fully dropped token gets y_shared
 * (or 0): the caller's residual connection carries it. */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* row_of,
                       const float* topk_w, const void* y_shared, void* y, void* stream);

/* Load statistics and balance loss ("Top-k 路由" 負載均衡 section;
 * "从 Dense FFN 到 MoE" §8; "别只比较 Top-k" [9,4,2,1] example):
 *   f[e]       = counts[e] / (T k)              (share of routed assignments)
 *   P[e]       = mean_t probs[t, e]             (importance)
 *   aux_loss   = alpha * E * sum_e f[e] P[e]    (= alpha for uniform routing)
 *   imbalance  = max_e counts[e] / (T k / E)
 *   dropped    = sum_e (counts[e] - min(counts[e], C))
 * counts [E] int32 and probs [T, E] float32 in; f, P [E], aux_loss [1],
 * imbalance [1] float32 and dropped [1] int32 out (each nullable).  Device
 * pointers.  ws: moe_workspace_size(MOE_OP_LOAD_STATS). */
moe_status moe_load_stats(const moe_config* cfg, const int32_t* counts, const float* probs,
                          float alpha, float* f, float* P, float* aux_loss, float* imbalance,
                          int32_t* dropped, void* ws, size_t ws_bytes, void* stream);

/* Layer weights (device pointers, act_dtype unless stated). */
typedef struct {
  const void* w_router;   /* [E, D] router_dtype */
  const float* sel_bias;  /* [E] float32, MOE_SIGMOID_BIAS only (NULL = zero) */
  const void* w13;        /* [E, 2F, D] SwiGLU or [E, F, D] GELU */
  const void* w2;         /* [E, D, F] */
  const void* ws13;       /* [2 S F_s, D] shared gate/up, concatenated; NULL iff S = 0 */
  const void* ws2;        /* [D, S F_s] shared down, concatenated */
} moe_weights;

/* Whole layer forward: route -> permute -> grouped expert FFN (reading x rows
 * through the permutation) -> shared experts -> combine (-> statistics).
 *   x [T, D] in; y [T, D] out (the branch output; the caller adds the residual)
 *   topk_idx [T, k], topk_w [T, k], counts [E]: optional outputs (NULL = skip)
 *   stats [2E + 2] float32 optional: f[0..E), P[E..2E), aux_loss, imbalance
 *   dropped [1] int32 optional
 *   alpha: balance-loss coefficient (used with stats)
 *   ws: moe_workspace_size(MOE_OP_LAYER) bytes.
 * Streams: work that does not lie on the routed path runs on a stream the
 * library creates once per device (default priority), forked from `stream`
 * with events and joined back to it: the shared experts' projections (they
 * need only x) from the start of the call, joined before the combine, and the
 * load statistics (they need the probabilities and counts) from the end of
 * the permutation, joined at the end of the call.  Every output is complete
 * when `stream` passes the call.  Calls from several host threads are
 * serialised around the forks and joins.  If a call fails after enqueueing,
 * work already enqueued on either stream may still run. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* weights,
                             const void* x, void* y, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, float alpha, float* stats, int32_t* dropped,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * arguments minus the workspace: the call runs in a scratch array that the
 * library holds in device memory, MOE_STATIC_SCRATCH_BYTES per GPU, kept
 * from the first call on a GPU until the process ends.  It allocates
 * nothing, creates no stream or event, and runs every kernel on `stream`
 * (the shared experts and the load statistics too, so nothing is forked).
 * A configuration whose moe_workspace_size(MOE_OP_LAYER) exceeds the scratch
 * is rejected with MOE_ERR_WORKSPACE_TOO_SMALL before any launch
 * (moe_last_error() names both sizes): 64 MiB holds decode-sized batches,
 * e.g. 256 tokens at the Mixtral- or DeepSeek-V3-shaped widths.  Every call
 * on one GPU uses the same scratch: calls that overlap on one GPU (two
 * streams, two host threads without ordering) race and must be serialised
 * by the caller.  Results equal moe_layer_forward's. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_static(const moe_config* cfg, const moe_weights* weights,
                                    const void* x, void* y, int32_t* topk_idx, float* topk_w,
                                    int32_t* counts, float alpha, float* stats, int32_t* dropped,
                                    void* stream);

/* Debug checks.  With the environment variable MOE_DEBUG=1 (read like the
 * tuning variables) the library copies the integer tables an entry point
 * reads or writes to the host, synchronising `stream`, and checks them
 * before it goes on; a table that breaks its definition fails the call with
 * MOE_ERR_DEBUG_CHECK and moe_last_error() names the first bad entry:
 *   moe_expert_ffn: offsets non-decreasing from >= 0 to <= max_rows, and
 *                   gather_rows[r] >= 0 for the rows the groups cover (before
 *                   any launch);
 *   moe_combine:    row_of in [-1, A_cap) (before any launch);
 *   moe_permute and the staged moe_layer_forward: counts, offsets, row_of
 *                   and token_of_row against the dispatch of topk_idx
 *                   ("从 Dense FFN 到 MoE" §5 batches, "Top-k 路由" 容量因子),
 *                   after the permutation.
 * Calls that synchronise cannot be captured in a HIP graph.
 *
 * moe_check_dispatch runs that dispatch check on HOST arrays (shapes as in
 * moe_permute): MOE_OK, or MOE_ERR_DEBUG_CHECK with the first difference in
 * moe_last_error().  For tools and tests; touches no device. */
moe_status moe_check_dispatch(const moe_config* cfg, const int32_t* topk_idx, const int32_t* counts,
                              const int32_t* offsets, const int32_t* row_of, const int32_t* token_of_row);

/* Re-reads the MOE_* tuning variables of the environment (tuning aids that
 * force a kernel choice: MOE_GEMM_CFG, MOE_GEMM_SPLIT, MOE_ROUTER_PATH, ...).
 * The library reads them once, at its first launch, and otherwise only here:
 * no launch path calls getenv.  For tuning tools and tests; not thread-safe
 * with respect to launches running on other host threads. */
moe_status moe_reload_tuning(void);

/* Kernel stages of moe_layer_forward, in launch order. */
typedef enum {
  MOE_STAGE_ROUTER_LOGITS = 0,   /* x W_g^T on the matrix cores / float32 ALUs */
  MOE_STAGE_ROUTE_SELECT = 1,    /* scoring, top-k, weights, probabilities */
  MOE_STAGE_PERMUTE = 2,         /* histogram, scan, scatter */
  MOE_STAGE_EXPERT_GATE_UP = 3,  /* grouped gate/up GEMM + activation */
  MOE_STAGE_EXPERT_DOWN = 4,     /* grouped down GEMM */
  MOE_STAGE_SHARED_GATE_UP = 5,
  MOE_STAGE_SHARED_DOWN = 6,
  MOE_STAGE_COMBINE = 7,
  MOE_STAGE_LOAD_STATS = 8,
  MOE_STAGE_FUSED_LAYER = 9,     /* every step above in one kernel (small batches) */
  MOE_NUM_STAGES = 10
} moe_stage;

/* Which stages moe_layer_forward runs for `cfg` in a call that asks for
 * every output: runs[s] = 1 or 0 for s < MOE_NUM_STAGES (host array).
 * Host-side only: no device is touched.  A small batch runs
 * MOE_STAGE_FUSED_LAYER alone: route, dispatch, experts, combine and
 * statistics in one launch of one workgroup per token, in which every
 * workgroup routes the whole batch and then runs its own token through its
 * experts.  Each step is defined as on the staged path (the logits and the
 * selection in double precision, the expert sums in float32 from the stored
 * values, the activations kept in float32 between the two projections).  It
 * runs when the batch fits (T <= 256, E <= 64, k <= 8; x, W_g, the float64
 * logits and the token's buffers within 63 KB of LDS) and the work of one
 * workgroup is small: T*E*D <= 262144 router multiply-adds and at most
 * 1048576 for the token's routed and shared experts.  The environment variable MOE_FUSED, read like the
 * other tuning variables (moe_reload_tuning), overrides the choice: 1 fuses
 * every batch that fits, 0 none. */
moe_status moe_layer_stages(const moe_config* cfg, int32_t* runs);

/* moe_layer_forward with stage timing: identical work, and for every stage s
 * that runs, hipEventRecord(stage_events[2s], <its stream>) before its kernels
 * and hipEventRecord(stage_events[2s+1], <its stream>) after them, where the
 * shared expert and load statistics stages run on the library's auxiliary
 * stream and the others on `stream`.  stage_events holds
 * 2 * MOE_NUM_STAGES caller-created hipEvent_t handles (entries may be NULL;
 * NULL array = no timing, i.e. moe_layer_forward).  For profiling tools. */
moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* weights,
                                   const void* x, void* y, int32_t* topk_idx, float* topk_w,
                                   int32_t* counts, float alpha, float* stats, int32_t* dropped,
                                   void* ws, size_t ws_bytes, void* stream,
                                   void* const* stage_events);

/* Backward pass of moe_layer_forward ("Top-k 路由" page, 門控網路的梯度流:
 * the gradient flows through the selected experts' gate scores, unselected
 * experts get none; "从 Dense FFN 到 MoE" §9: selected experts get the task
 * gradient, the router gets it through the selected route weights and the
 * balance loss's gradient through the soft importance).  The loss is
 *   <dy, y> + L_aux,   L_aux = alpha * E * sum_e f_e P_e
 * with the routing decisions (expert ids, capacity drops, the counts behind
 * f) held fixed.  The call recomputes the forward (routing, permutation and
 * the expert activations, in its workspace) and returns:
 *   dx        [T, D] act_dtype out
 *   dw_router [E, D] float32 out
 *   dw13      [E, n_mat F, D] float32 out (rows as w13: SwiGLU gate then up)
 *   dw2       [E, D, F] float32 out
 *   dws13     [2 S F_s, D] float32 out, dws2 [D, S F_s] float32 out (NULL
 *             iff S = 0)
 * Experts without rows get zero gradients.  act_dtype must be MOE_BF16
 * (MOE_ERR_UNSUPPORTED otherwise); intermediates are bf16 with float32
 * accumulation.  ws: moe_workspace_size(MOE_OP_LAYER_BACKWARD) bytes (it holds
 * transposed copies of the expert weights).  Deterministic. */
moe_status moe_layer_backward(const moe_config* cfg, const moe_weights* weights, const void* x, const void* dy,
                              float alpha, void* dx, float* dw_router, float* dw13, float* dw2, float* dws13,
                              float* dws2, void* ws, size_t ws_bytes, void* stream);

/* Expert-choice routing ("Top-k 路由" page, Token-Choice vs Expert-Choice
 * table: each expert picks its top-C tokens; "MoE 路由算法" page, 数学机理
 * (2), and 深度剖析 ② on tokens no expert picks).  The layer forward with the
 * routing reversed:
 *   p = softmax(W_g x) over the experts (float32, from the router logits);
 *   expert e takes the C tokens with the largest p[:, e] (equal values: the
 *   lower token index first), gate p[t, e];
 *   C = ceil(CF * T * k / E) (the buffer formula of the 容量因子 section; k =
 *   cfg->top_k read as the average experts per token, CF =
 *   cfg->capacity_factor, or 1 when <= 0), at most T: moe_expert_choice_capacity;
 *   rows expert after expert, tokens ascending inside an expert (E * C rows);
 *   the grouped expert FFN of cfg->activation on the rows, the shared experts
 *   (weight 1, every token) as in moe_layer_forward;
 *   y[t] = sum over the experts that took t, ascending, of p[t, e] *
 *   FFN_e(x[t]) (+ shared); a token no expert took gets only the shared
 *   output (0 without shared experts): the caller's residual carries it.
 * cfg->scoring and cfg->renormalize are not used.  Limits: E <= 256,
 * T <= 8192 (MOE_ERR_UNSUPPORTED beyond).
 *   x, y           [T, D] act_dtype device
 *   token_of_row   [E * C] int32 out or NULL; row_w [E * C] float32 out or NULL
 *   unselected     [1] int32 out or NULL: tokens no expert took
 *   ws             moe_workspace_size(MOE_OP_EXPERT_CHOICE) bytes
 *   stage_events   NULL, or 2 * MOE_NUM_STAGES hipEvent_t as for
 *                  moe_layer_forward_timed (route: ROUTER_LOGITS and
 *                  ROUTE_SELECT; PERMUTE and LOAD_STATS are not used)
 * Bit-exact choices (outside near ties of p) and deterministic outputs. */
moe_status moe_expert_choice_capacity(const moe_config* cfg, int32_t* capacity);
moe_status moe_expert_choice_forward(const moe_config* cfg, const moe_weights* weights, const void* x, void* y,
                                     int32_t* token_of_row, float* row_w, int32_t* unselected,
                                     void* ws, size_t ws_bytes, void* stream, void* const* stage_events);

/* Expert parallelism, the part one GPU holds ("Top-k 路由" page, 通訊拓撲：
 * All-to-All figure; "别只比较 Top-k" page, two-All-to-All dispatcher and
 * 按目标专家发送 sections).  Experts sit on ranks in contiguous blocks of
 * E / R; the exchanges themselves (all-to-all over the interconnect) are the
 * caller's.
 *
 * Send layout: with the rows of moe_permute (expert-major), the rows bound for
 * rank r are the contiguous run send_offsets[r] .. send_offsets[r+1]:
 *   offsets      [E+1] int32 device in (moe_permute's)
 *   send_counts  [R] int32 device out: kept rows of rank r's experts
 *   send_offsets [R+1] int32 device out: exclusive prefix of send_counts
 * num_experts % num_ranks == 0, 1 <= num_ranks <= num_experts. */
moe_status moe_ep_send_layout(int32_t num_experts, int32_t num_ranks, const int32_t* offsets,
                              int32_t* send_counts, int32_t* send_offsets, void* stream);

/* Receive layout: the exchange delivers the sources one after another, each
 * source's rows expert after expert.  The local grouped FFN reads them expert
 * after expert (sources in rank order inside an expert) through a gather map,
 * with no copy: moe_expert_ffn(num_groups = local_experts, x_in = received
 * rows, gather_rows = gather, offsets = local_offsets).
 *   recv_counts   [R, E_local] int32 device in: rows source r sends for local
 *                 expert e (what the count exchange delivers)
 *   rows_cap      capacity of gather (>= the received total, which the
 *                 caller knows after the count exchange; rows past rows_cap
 *                 are not described and local_offsets are clamped to it)
 *   local_offsets [E_local+1] int32 device out
 *   gather        [rows_cap] int32 device out: received position of
 *                 expert-major row j; -1 past the received total
 * Bit-exact and deterministic. */
moe_status moe_ep_recv_layout(int32_t num_ranks, int32_t local_experts, const int32_t* recv_counts,
                              int32_t rows_cap, int32_t* local_offsets, int32_t* gather, void* stream);

/* Static text of a status code; the last HIP error text of this thread. */
const char* moe_status_string(moe_status status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
