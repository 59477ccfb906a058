/*
 * moe.h -- C ABI of the routed Mixture-of-Experts SwiGLU feed-forward layer
 * for AMD Instinct MI355X (gfx950): forward and backward on one GPU's share
 * of a packed token batch.
 *
 * What the layer computes (the sources are three public pages about small-lab
 * decoder-only LM training, cited by title and section):
 *   - KochiLLM v1.0 model card, "Architecture": an always-on shared expert
 *     plus the top-2 of 4 routed experts per token, the two routing weights
 *     rescaled to sum to one, and the balancing term 4 * sum_i f_i * p_i.
 *   - spark-gpt README, feature list (optional Qwen3-MoE layers): router
 *     without bias, softmax in fp32, top-k, SwiGLU experts with gate and up
 *     weights packed in one tensor, rescaling of the chosen probabilities
 *     (optional, MoE paragraph), the balancing statistic from integer counts
 *     and a differentiable probability mean, plus router metrics.
 *   - KohakUwULLM README, "Key features": MXFP8 experts (e4m3 values, one
 *     power-of-two UE8M0 scale per 32 elements).
 *
 * Conventions shared by every call
 *   - Every pointer argument is DEVICE memory unless stated otherwise.  The
 *     caller allocates and frees all of it, including the workspace whose
 *     size moe_workspace_bytes() returns.  The library never allocates on
 *     the compute calls and keeps no pointer past a call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every compute
 *     call only enqueues work on that stream and returns; nothing
 *     synchronises with the host and no data-dependent size leaves the GPU.
 *   - "act" below is the plan's activation dtype (f32, f16 or bf16): x, y,
 *     dy, dx, the router weight and the expert weights are stored in it, and
 *     so are H and the weight gradients.  A bf16 layer with bf16 experts keeps
 *     three intermediates in f32: the saved gate/up pre-activations GU, the
 *     expert outputs Y_perm and (in the workspace) the experts' input-gradient
 *     rows; rounded to bf16 they alone move y, dx and the router gradient by
 *     2-3 % of their RMS at 16k tokens x top-8.  f16 and f32 layers keep them
 *     in act.  With MX-fp8 experts GU is bf16 and Y_perm f32 (the
 *     routing-weight gradient is taken from Y_perm there).  Router
 *     probabilities and routing weights are always f32.
 *     Every matrix is row-major with the last index contiguous.
 *   - Arguments are checked on the host before anything is launched; a
 *     negative moe_status is returned and nothing is enqueued.  A HIP launch
 *     error is reported as MOE_ERR_HIP.  Device-side preconditions (indices
 *     in range, each token's k experts distinct) are documented per call and
 *     not checked on the device; kernels never write outside the buffers
 *     the sizes describe even when they are violated.
 *   - A plan is immutable after creation except for the optional kernel
 *     timing probe (moe_probe_*), which is not thread-safe.  Calls on
 *     different streams may share a plan if each uses its own workspace.
 *   - No float atomics are used: two runs on the same inputs give bitwise
 *     identical results.
 */
#ifndef MOE_FFN_MI355X_H
#define MOE_FFN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_INVALID = -2,     /* a size or flag is out of range */
  MOE_ERR_UNSUPPORTED = -3, /* valid but not implemented (dtype pair, alignment) */
  MOE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -5,         /* the HIP runtime reported an error */
  MOE_ERR_SCRATCH = -6      /* an allocation-free call needs more than its fixed scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_F16 = 1, MOE_BF16 = 2, MOE_MXFP8_E4M3 = 3 } moe_dtype;

/* Layer shape.  Requirements checked by moe_plan_create():
 *   0 <= T;  1 <= top_k <= n_experts <= 256;
 *   d_model, d_ff (and d_ff_shared when n_shared > 0) multiples of 128;
 *   0 <= n_shared <= 8;  act_dtype in {F32, F16, BF16};
 *   expert_dtype == act_dtype, or expert_dtype == MXFP8_E4M3 with act_dtype
 *   BF16 (the MX GEMMs write bf16): then every expert GEMM (routed and shared, forward and
 *   backward) quantises both operands to MX-fp8 along that GEMM's reduction
 *   axis (blocks of 32; along the tokens of each expert segment for the
 *   weight gradients) into the workspace and runs on the scaled fp8 matrix
 *   cores; weights, activations, gradients and outputs stay in act_dtype.
 *   The router, softmax, combine and statistics are never quantised.
 *   (KohakUwULLM README, "Key features": MXFP8 experts.) */
typedef struct {
  int64_t T;              /* tokens in the packed batch (rows of x) */
  int32_t d_model;        /* d */
  int32_t n_experts;      /* E routed experts */
  int32_t top_k;          /* k experts per token */
  int32_t d_ff;           /* I, inner width of a routed expert */
  int32_t n_shared;       /* Ns always-on shared experts (0 = none) */
  int32_t d_ff_shared;    /* Is, inner width of a shared expert */
  int32_t renorm;         /* 1: routing weights = chosen probs / their sum; 0: chosen probs */
  int32_t has_router_bias;/* 1: moe_route adds a constant f32 bias[E] to the logits */
  int32_t act_dtype;      /* moe_dtype */
  int32_t expert_dtype;   /* moe_dtype of the expert GEMM operands */
  float aux_coef;         /* alpha: coefficient of the balancing statistic in the loss */
  int32_t router;         /* moe_router: how moe_route chooses and weights the experts */
  int32_t mx_fused;       /* MX-fp8 plans, 1: only the fused path (KohakUwULLM README, "Key
                             features": fused MXFP8 experts without the (tokens x top_k, hidden)
                             intermediates): the workspace then holds neither the act-dtype
                             dY_perm and [dG | dU] rows nor the backward's own codes of the
                             weights and H, and the x codes only for the T rows; every
                             moe_expert_ffn / moe_backward call must then pass perm_token and
                             mx_saved (MOE_ERR_NULL otherwise), and moe_keep_intermediates is
                             refused (MOE_ERR_UNSUPPORTED).  Needs T * d_model < 2^31.  0: both
                             paths (the default).  Must be 0 for other plans. */
} moe_config;

/* Router kinds (moe_config.router).
 * MOE_ROUTER_SOFTMAX: f32 softmax over the experts, top-k (spark-gpt README,
 *   feature list); moe_route_balanced and moe_route_sinkhorn are its variants.
 * MOE_ROUTER_RELU: the ReLU router (KohakUwULLM README, "Key features": ReLU
 *   routers beside the default; the pages give no rule, so this library
 *   follows the published ReLU routing): gates g = max(z, 0) with z the
 *   logits (+ bias), no softmax; each token takes its experts with a positive
 *   logit, at most top_k of them (the largest, descending, lower index first
 *   on ties); the remaining slots hold index -1 and weight 0 and are no
 *   assignment (moe_permute skips them, so offsets[E] <= T*k); the weights
 *   are the gates themselves (cfg.renorm must be 0); probs holds the gates,
 *   so the balancing statistic E sum_e f_e mean_t g_te is the published
 *   load-balanced L1 term on them; moe_backward applies dz = dg where the
 *   gate is positive, 0 elsewhere.
 * MOE_ROUTER_EXPERT_CHOICE: the expert-choice router (KohakUwULLM README,
 *   "Key features": expert-choice routers beside the default; the pages give
 *   no rule, so this library follows the published method), routed with
 *   moe_route_expert_choice (moe_route refuses it): every expert takes the
 *   C = T top_k / E (rounded down) tokens of largest f32 softmax probability
 *   (lower token index first on ties), so a token is taken by 0 to E experts.
 *   The routing arrays then have one slot per expert: topk_idx, topk_w and
 *   inv_perm are [T, E] (slot e holds e or -1, the weight the probability or
 *   0; cfg.renorm must be 0), everything [T, k]-shaped elsewhere in this
 *   header is [T, E], and E <= 64 (MOE_ERR_UNSUPPORTED otherwise); rows stay
 *   at most T top_k (E C of them), and the statistic's f_e = count_e /
 *   (T top_k) = C / (T top_k), the same for every expert.  moe_backward
 *   applies the softmax Jacobian to the taken slots' gradients (the choice
 *   carries no gradient). */
typedef enum { MOE_ROUTER_SOFTMAX = 0, MOE_ROUTER_RELU = 1, MOE_ROUTER_EXPERT_CHOICE = 2 } moe_router;

typedef struct moe_plan_s* moe_plan;

/* Validate `cfg` and build a plan (host memory only; selects every kernel
 * variant once).  *out is set to NULL on failure.  The GEMM tile sizes may be
 * forced for tuning with the environment variables MOE_ROW_TILE and
 * MOE_WGRAD_TILE (128 or 256), read here; a value the shape does not allow
 * is ignored.  Results do not depend on the tile size beyond f32 rounding
 * order within a tile's K loop, which is the same for both sizes. */
moe_status moe_plan_create(const moe_config* cfg, moe_plan* out);
void moe_plan_destroy(moe_plan plan);
/* Bytes of device workspace the compute calls need (same for all calls). */
size_t moe_workspace_bytes(moe_plan plan);
/* Bytes of the optional MX-fp8 saved-codes buffer (moe_ffn_args.mx_saved);
 * 0 for a NULL plan or a plan without MX-fp8 experts. */
size_t moe_mx_saved_bytes(moe_plan plan);
/* Static description of a status code. */
const char* moe_status_string(moe_status status);
/* Library version string, e.g. "moe-ffn-mi355x 0.1 gfx950". */
const char* moe_version(void);

/* ---- forward ----------------------------------------------------------- */

/* Router: z = x W_r^T (+ bias); probs = softmax(z) in f32 (max-subtracted);
 * topk_idx[t, :] = the k largest logits, ordered by logit descending and, on
 * equal logits, by lower expert index; topk_w = the chosen probs, divided by
 * their sum when cfg.renorm.  (spark-gpt feature list; KochiLLM
 * "Architecture".)
 *   x         [T, d] act          w_router [E, d] act
 *   bias      [E] f32, required iff cfg.has_router_bias, else ignored
 *   probs     [T, E] f32 out      topk_idx [T, k] int32 out   topk_w [T, k] f32 out */
moe_status moe_route(moe_plan plan, const void* x, const void* w_router, const float* bias,
                     float* probs, int32_t* topk_idx, float* topk_w, void* stream);

/* Router with aux-loss-free load balancing (KohakUwULLM README, "Key
 * features": DeepSeekMoE with aux-loss-free load balancing; the pages give no
 * rule, so this library follows the published method).  As moe_route, except
 * that the experts are ranked on probs[t, e] + sel_bias[e], computed in f32
 * (descending; on equal values the lower expert index first), while topk_w
 * still holds the unbiased probabilities of the chosen experts (divided by
 * their sum when cfg.renorm).  The selection bias carries no gradient, and
 * moe_backward needs nothing else: it reads the chosen indices and weights.
 *   sel_bias  [E] f32 in (required)
 *   other arguments as for moe_route. */
moe_status moe_route_balanced(moe_plan plan, const void* x, const void* w_router, const float* bias,
                              const float* sel_bias, float* probs, int32_t* topk_idx, float* topk_w,
                              void* stream);

/* Expert-choice router (see MOE_ROUTER_EXPERT_CHOICE; the plan must have that
 * router): probs as moe_route, then every expert takes its C tokens of
 * largest probability by a radix select on the f32 bit patterns of its
 * column, deterministically (no float atomics).
 *   topk_idx  [T, E] int32 out: e where expert e took token t, else -1
 *   topk_w    [T, E] f32 out: probs[t, e] where taken, else 0
 *   ws        the plan's workspace (it holds the transposed probabilities)
 *   other arguments as for moe_route. */
moe_status moe_route_expert_choice(moe_plan plan, const void* x, const void* w_router, const float* bias,
                                   float* probs, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                                   void* stream);

/* Sinkhorn router (KohakUwULLM README, "Key features": Sinkhorn routers
 * beside the default; the pages give no rule, so this library follows the
 * published Sinkhorn-Knopp balancing of the batch's routing probabilities).
 * probs as moe_route; then n_iter rounds of
 *   a_t = (1/T) / sum_e probs[t, e] b_e,   b_e = (1/E) / sum_t probs[t, e] a_t
 * from b = 1 (f32, every sum in a fixed order), and each token's k experts
 * are the largest probs[t, e] * b_e (descending; on equal values the lower
 * expert index first).  topk_w holds the chosen probabilities themselves
 * (divided by their sum when cfg.renorm): the selection carries no gradient
 * and moe_backward runs as for moe_route.  No host synchronisation: the
 * rounds are a fixed count of launches.
 *   n_iter    rounds, 1 .. 1000 (MOE_ERR_INVALID otherwise)
 *   col_scale [E] f32 out: b after the last round
 *   ws        the plan's workspace (moe_workspace_bytes); E <= 256
 *   other arguments as for moe_route. */
moe_status moe_route_sinkhorn(moe_plan plan, const void* x, const void* w_router, const float* bias,
                              int32_t n_iter, float* probs, int32_t* topk_idx, float* topk_w, float* col_scale,
                              void* ws, size_t ws_bytes, void* stream);

/* The step-end update of the selection bias (same reading as above):
 * sel_bias[e] += gamma * sign(T k - E counts[e]), i.e. a fixed step down for
 * experts above the mean load T k / E and up for those below; the sign is
 * decided exactly in integers and the addition rounds once in f32.
 *   counts    [E] int32 in (the step's expert loads, e.g. from moe_permute)
 *   sel_bias  [E] f32 in/out
 *   gamma     >= 0 and finite, else MOE_ERR_INVALID. */
moe_status moe_balance_update(moe_plan plan, const int32_t* counts, float* sel_bias, float gamma, void* stream);

/* Group the T*k assignments by expert, stably (expert ascending, then token
 * ascending), and gather the token rows in that order.
 *   topk_idx   [T, k] int32 in: values in [0, E), distinct within a row
 *   x          [T, d] act in
 *   counts     [E] int32 out: assignments per expert
 *   offsets    [E+1] int32 out: exclusive prefix sum of counts (offsets[E] = T*k)
 *   perm_token [T*k] int32 out: token of each expert-sorted row
 *   inv_perm   [T, k] int32 out: expert-sorted row of assignment (t, j)
 *   x_perm     [T*k, d] act out: x_perm[r] = x[perm_token[r]]; or NULL (then x may be
 *              NULL too): only the indices are produced, for MX-fp8 plans whose
 *              expert GEMMs gather x's rows by perm_token */
moe_status moe_permute(moe_plan plan, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* inv_perm, void* x_perm,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and error checks as
 * moe_permute; its scratch (2 * ceil(T / 256) * E int32, each half rounded up
 * to 256 bytes) lives in a fixed 1 MiB device array inside the library, one
 * per GPU, held until the process ends; a plan needing more returns
 * MOE_ERR_SCRATCH before anything is launched (e.g. T <= 65536 with E <= 256
 * fits).  Nothing in the scratch has to start at zero (every call writes what
 * it reads).  The first call on a device looks up the array's address
 * (hipGetSymbolAddress); no call allocates.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (concurrent streams, or
 * threads) race and must be ordered by the caller. */
moe_status moe_permute_noalloc(moe_plan plan, const int32_t* topk_idx, const void* x, int32_t* counts,
                               int32_t* offsets, int32_t* perm_token, int32_t* inv_perm, void* x_perm,
                               void* stream);

/* Pointers of the expert FFN (shared-expert fields are ignored when n_shared == 0). */
typedef struct {
  const void* x_perm;      /* [T*k, d] act, rows grouped by expert */
  const int32_t* offsets;  /* [E+1] from moe_permute */
  const void* w_gate_up;   /* [E, 2I, d] act: rows 0..I-1 gate, I..2I-1 up */
  const void* w_down;      /* [E, d, I] act */
  void* gu;                /* out [T*k, 2I]: [G | U] per row, saved for backward; f32 for a
                              bf16 layer with bf16 experts, bf16 for MX-fp8 experts, else act */
  void* h;                 /* out [T*k, I] act: silu(G) * U (MX-fp8 plans given mx_saved: may be
                              NULL, H then exists only as its two MX codes) */
  void* y_perm;            /* out [T*k, d]: H W_d^T; f32 for a bf16 layer with bf16 experts, else act */
  const void* x;           /* [T, d] act (shared experts' input) */
  const void* ws_gate_up;  /* [Ns, 2Is, d] act */
  const void* ws_down;     /* [Ns, d, Is] act */
  void* gu_shared;         /* out [T, 2 Ns Is], dtype as gu: expert s in columns [2 s Is, 2 (s+1) Is) as [G_s | U_s] */
  void* h_shared;          /* out [T, Ns Is] act: expert s in columns [s Is, (s+1) Is) (NULL as h) */
  void* y_shared;          /* out [T, d] act: sum over shared experts */
  /* Optional, MX-fp8 plans: perm_token [T*k] from moe_permute.  Given it,
   * the gate/up GEMM gathers its rows on load from x quantised once per
   * token (x must then be set) instead of quantising the T*k rows of x_perm;
   * x_perm is not read.  NULL keeps the x_perm path.  Ignored otherwise. */
  const int32_t* perm_token;
  /* Optional, MX-fp8 plans: a buffer of moe_mx_saved_bytes() bytes that the
   * forward fills with operand codes the backward would otherwise make
   * (pass it on as moe_saved.mx_saved): the weights' codes along the
   * backward's reduction axes (W_gu along 2 d_ff, W_d along d, the shared
   * experts' likewise), written by the same pass that reads the weights for
   * the forward's codes, and H's codes along each expert's tokens (and the
   * shared experts' H along the T tokens), written by the gate/up epilogue
   * beside H.  NULL: the backward quantises them itself.  Ignored otherwise. */
  void* mx_saved;
} moe_ffn_args;

/* Routed experts as grouped GEMMs over the expert segments of x_perm (gate/up
 * GEMM with SwiGLU in its epilogue, then the down GEMM), plus the shared
 * experts on all T rows.  No biases.  (KochiLLM "Configuration"/"Architecture";
 * spark-gpt feature list.) */
moe_status moe_expert_ffn(moe_plan plan, const moe_ffn_args* args, void* ws, size_t ws_bytes,
                          void* stream);

/* y[t] = sum_j topk_w[t, j] * y_perm[inv_perm[t, j]] (+ y_shared[t]), accumulated in
 * f32 in slot order j = 0..k-1, one write per row.
 *   y_perm [T*k, d], dtype as in moe_ffn_args; inv_perm [T, k] int32; topk_w [T, k] f32;
 *   y_shared [T, d] act or NULL; y [T, d] act out. */
moe_status moe_combine(moe_plan plan, const void* y_perm, const int32_t* inv_perm,
                       const float* topk_w, const void* y_shared, void* y, void* stream);

/* ---- backward ---------------------------------------------------------- */

/* Tensors saved by the forward (all produced by the calls above or inputs to them). */
typedef struct {
  const void* x;            /* [T, d] */
  const void* w_router;     /* [E, d] */
  const float* probs;       /* [T, E] */
  const int32_t* topk_idx;  /* [T, k] */
  const float* topk_w;      /* [T, k] */
  const int32_t* counts;    /* [E] */
  const int32_t* offsets;   /* [E+1] */
  const int32_t* inv_perm;  /* [T, k] */
  const void* x_perm;       /* [T*k, d] */
  const void* gu;           /* [T*k, 2I], dtype as in moe_ffn_args */
  const void* h;            /* [T*k, I] (not read, may be NULL, with mx_saved) */
  const void* y_perm;       /* [T*k, d], dtype as in moe_ffn_args (read for MX-fp8 experts only) */
  const void* w_gate_up;    /* [E, 2I, d] */
  const void* w_down;       /* [E, d, I] */
  const void* ws_gate_up;   /* [Ns, 2Is, d] (n_shared > 0) */
  const void* ws_down;      /* [Ns, d, Is] */
  const void* gu_shared;    /* [T, 2 Ns Is] */
  const void* h_shared;     /* [T, Ns Is] (not read, may be NULL, with mx_saved) */
  /* Balancing statistic over real tokens only (spark-gpt MoE paragraph):
   * real_mask [T] int32 (0 = filler) and real_counts [E+1] from
   * moe_aux_stats_masked of the same step; NULL real_mask = every token. */
  const int32_t* real_mask;
  const int32_t* real_counts;
  /* perm_token [T*k] from moe_permute.  Required unless the experts are
   * MX-fp8: the down projection's input gradient reads dy's rows through
   * it.  Optional for MX-fp8 plans: given it, the weight gradient of the
   * gate/up projection gathers x's rows by it instead of reading x_perm
   * (which may then be NULL). */
  const int32_t* perm_token;
  /* Optional, MX-fp8 plans: the moe_ffn_args.mx_saved buffer the forward of
   * this step filled (the weights unchanged since).  NULL: the backward
   * quantises the weights and H itself.  Ignored otherwise. */
  const void* mx_saved;
} moe_saved;

/* Gradient outputs (act dtype unless noted).  Every weight gradient is fully
 * written, including zeros for experts that received no token. */
typedef struct {
  void* dx;            /* [T, d] */
  void* dw_router;     /* [E, d] */
  float* dbias;        /* [E] f32: sum_t dL/dz_te, or NULL (the bias is a constant input) */
  void* dw_gate_up;    /* [E, 2I, d] */
  void* dw_down;       /* [E, d, I] */
  void* dws_gate_up;   /* [Ns, 2Is, d] (n_shared > 0) */
  void* dws_down;      /* [Ns, d, Is] */
} moe_grads;

/* Gradients of L = <dy, y> + aux_coef * aux with respect to x and every
 * weight.  The counts f_e carry no gradient; P_e = mean_t probs[t, e] does
 * (spark-gpt MoE paragraph).  With renorm the routing-weight gradient goes
 * through the division by the chosen-probability sum; the softmax Jacobian
 * is applied in f32.  The routing-weight gradient g[t, j] = <dy_t, Y_perm
 * row> is formed as <dy_t W_d, H> from the saved G, U (so Y_perm is not
 * read), except with MX-fp8 experts, whose g is <dy_t, Y_perm row>.
 * Rounding of the expert weight gradients' operands (bf16 / f32 layers): the
 * down weight gradient pairs dy's own rows with w H formed in f32 and rounded
 * once; with fewer than 128 rows per expert on average (bf16), both expert
 * weight gradients also add the products of the operands' rounding
 * remainders (one more GEMM pass each), since a gradient element summed over
 * a handful of rows shows a single bf16 rounding undamped.
 *   dy [T, d] act in.
 * Plans with 16-bit or f32 experts need T * d_model * (element bytes) < 2^31
 * (moe_plan_create returns MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_backward(moe_plan plan, const moe_saved* saved, const void* dy,
                        const moe_grads* grads, void* ws, size_t ws_bytes, void* stream);

/* ---- balancing statistic and router metrics ---------------------------- */

typedef struct {
  float aux;           /* E * sum_e f_e P_e (1 at perfect balance) */
  float aux_raw;       /* sum_e f_e P_e */
  float entropy_mean;  /* mean_t of -sum_e p_te ln p_te */
  float count_cv;      /* population std / mean of counts */
  int32_t count_min;
  int32_t count_max;
  int32_t n_unused;    /* experts with count 0 */
  int32_t reserved;
} moe_aux_scalars;

/* f_e = counts[e] / (T k); P_e = mean_t probs[t, e]; and the scalars above
 * (KochiLLM "Architecture" for the statistic; spark-gpt MoE paragraph for the
 * metrics).  Reductions run in a fixed order.
 *   probs [T, E] f32; counts [E] int32; f, p_mean [E] f32 out;
 *   out: one moe_aux_scalars in DEVICE memory. */
moe_status moe_aux_stats(moe_plan plan, const float* probs, const int32_t* counts, float* f,
                         float* p_mean, moe_aux_scalars* out, void* ws, size_t ws_bytes,
                         void* stream);

/* The same statistic over the real tokens only, fillers (padding) left out
 * (spark-gpt README, MoE paragraph: the statistic is computed over real,
 * non-filler tokens).  With T_r = the number of tokens whose mask is non-zero:
 * real_counts[e] = assignments of real tokens to e, real_counts[E] = T_r,
 * f_e = real_counts[e] / (T_r k), P_e = the mean of probs[t, e] over real t,
 * and every metric taken over the real tokens; T_r = 0 gives zeros.
 * moe_backward applies the statistic's gradient to real tokens only when
 * moe_saved.real_mask and .real_counts are set from this call.
 *   probs [T, E] f32; topk_idx [T, k] int32; real_mask [T] int32;
 *   f, p_mean [E] f32 out; real_counts [E+1] int32 out;
 *   out: one moe_aux_scalars in DEVICE memory. */
moe_status moe_aux_stats_masked(moe_plan plan, const float* probs, const int32_t* topk_idx,
                                const int32_t* real_mask, float* f, float* p_mean, int32_t* real_counts,
                                moe_aux_scalars* out, void* ws, size_t ws_bytes, void* stream);

/* ---- MX-fp8 quantisation ----------------------------------------------- */

/* Quantise `rows` rows of K values (act_dtype BF16 or F16, row-major, K a
 * multiple of 32) to MX-fp8 along the row: per block of 32 values the scale is
 * the smallest power of two 2^x with max|v| <= 448 * 2^x (x clamped to
 * [-127, 127]; -127 for an all-zero block), scales[r * K/32 + b] = x + 127
 * (UE8M0), and payload[r * K + k] = v / 2^x rounded to nearest OCP e4m3 (ties
 * to even; subnormals k * 2^-9).  The quantiser the MX expert GEMMs use, as a
 * call of its own.  (KohakUwULLM README, "Key features": e4m3 values with one
 * power-of-two scale per 32 elements; the choice of the scale is this
 * library's reading: no value saturates.)
 *   in       [rows, K] act          payload [rows, K] bytes
 *   scales   [rows, K/32] bytes
 * Returns MOE_ERR_NULL / MOE_ERR_INVALID before any launch on bad arguments. */
moe_status moe_mx_quantize_rows(const void* in, int32_t act_dtype, int64_t rows, int32_t K, uint8_t* payload,
                                uint8_t* scales, void* stream);

/* ---- kernel timing probe (measurement aid) ----------------------------- */

/* Record a hipEvent pair around each of the next `max_launches` launches of
 * the kernel named `kernel` (see moe_kernel_names()) on the stream it runs
 * on.  max_launches <= 0 disables the probe.  Creates events (host call). */
moe_status moe_probe_enable(moe_plan plan, const char* kernel, int max_launches);
/* Synchronise the recorded events and return the sum of their durations and
 * how many launches were recorded; resets the probe. */
moe_status moe_probe_read(moe_plan plan, float* total_ms, int* launches);
/* Comma-separated names of the kernels the probe accepts. */
const char* moe_kernel_names(void);

/* ---- backward intermediates (inspection aid) --------------------------- */

/* Byte offset and size, inside the workspace, of an intermediate that
 * moe_backward keeps there and leaves in place when it returns (until the
 * next call that uses the workspace), row-major, act dtype except dx_perm and
 * dx_shared, which are f32 in a bf16 layer with bf16 experts:
 *   "dy_perm"     [T*top_k, d_model]     gradient reaching the expert rows:
 *                 w dy (f16 layers, MX-fp8 experts) or dy itself (bf16 and
 *                 f32 layers, whose routing weight sits in "wh")
 *   "wh"          [T*top_k, d_ff]        bf16 / f32 layers: the routing weight
 *                 times H = silu(G) U formed from the saved G, U, the down
 *                 weight gradient's other operand
 *   "dgu_lo", "wh_lo"  (bf16 plans whose experts see fewer than 128 rows on
 *                 average) the rounding remainders v - bf16(v) of "dgu" and
 *                 "wh", in bf16, which the expert weight gradients add
 *   "dgu"         [T*top_k, 2 d_ff]      [dG | dU] of the routed experts
 *                 (MX-fp8 plans: only after moe_keep_intermediates(plan, 1),
 *                 as "dgu_shared", and "dy_perm" when the backward was given
 *                 perm_token)
 *   "dx_perm"     [T*top_k, d_model]     input gradient of the expert rows
 *   "dgu_shared"  [T, 2 n_shared d_ff_shared]  [dG_s | dU_s] per shared expert
 *   "dx_shared"   [T, d_model]           input gradient of the shared experts
 * Plans with MX-fp8 experts also expose the quantised operand of every
 * expert GEMM, each as "<name>" (e4m3 payload bytes, [rows][K]) and
 * "<name>.scales" (UE8M0 bytes = exponent + 127, [rows][K/32]), blocks of 32
 * along K; A = T*top_k, Apad = the expert segments' token counts rounded up
 * to multiples of 128 and summed (plus headroom), Tpad = T rounded up to 128,
 * NI = n_shared * d_ff_shared:
 *   row operands (K = the contraction of the GEMM reading them)
 *   "mx_xq"   [A][d]       x_perm (x_perm path) or x's T rows (gather path,
 *                          routed experts only)
 *   "mx_hq"   [A][d_ff]    H (written by the gate/up epilogue)
 *   "mx_dyq"  [A][d]       dY_perm (written by the combine backward)
 *   "mx_dguq" [A][2 d_ff]  [dG | dU] (written by the SwiGLU-backward epilogue)
 *   "mx_wgu"  [E 2 d_ff][d]   "mx_wd" [E d][d_ff]   expert weights
 *   "mx_wdt"  [d_ff][E d]     "mx_wgut" [d][E 2 d_ff]  weights along d / 2 d_ff
 *   token-axis operands of the weight gradients ([C][Apad]; expert e's tokens
 *   at K positions mx_pad[e] .. mx_pad[e] + count_e, blocks of 32 restarting
 *   at mx_pad[e], zeros up to mx_pad[e+1])
 *   "mx_dyt" [d][Apad]  "mx_ht" [d_ff][Apad]  "mx_dgut" [2 d_ff][Apad]  "mx_xt" [d][Apad]
 *   "mx_pad" [E+1] int32, the padded segment starts
 *   shared experts (n_shared > 0): "mx_sxq" [T][d] (x, also read by the routed
 *   experts on the gather path), "mx_shq" [T][NI], "mx_sdyq" [T][d] (dY),
 *   "mx_sdguq" [T][2 NI], "mx_swgu" [2 NI][d], "mx_swd" [d][NI],
 *   "mx_swdt" [NI][d], "mx_swgut" [d][2 NI], and token-axis (one segment of
 *   T tokens, zeros up to Tpad) "mx_sdyt" [d][Tpad], "mx_sht" [NI][Tpad],
 *   "mx_sdgut" [2 NI][Tpad], "mx_sxt" [d][Tpad].
 * Each holds what the last call that wrote it left there.
 * For tests and debugging, e.g. to check each GEMM of the backward on its
 * own inputs.  MOE_ERR_NULL for a null argument, MOE_ERR_INVALID for an
 * unknown name or a region this plan does not have (no shared experts, not
 * an MX plan; a fused-only plan has no "dy_perm", "dgu", "dgu_shared" and
 * none of "mx_wdt", "mx_wgut", "mx_ht" and their shared counterparts, which
 * its saved-codes buffer holds, and its "mx_xq" has T rows). */
moe_status moe_workspace_region(moe_plan plan, const char* name, size_t* offset, size_t* bytes);

/* MX-fp8 plans: the backward reads [dG | dU] (routed and shared) only through
 * the two MX operands the SwiGLU-backward epilogue writes ("mx_dguq",
 * "mx_dgut" and their shared counterparts), so by default it does not also
 * store the act-dtype "dgu" and "dgu_shared" rows (T*top_k * 2 d_ff * 2 bytes
 * of HBM writes saved); given moe_saved.perm_token, the same holds for the
 * "dy_perm" rows (their row-wise codes come from the combine backward, their
 * token-axis codes from dy's rows gathered by perm_token and scaled by the
 * routing weight as the rows would be).  keep = 1 makes later moe_backward
 * calls on this plan store them too, for tests and debugging; keep = 0
 * restores the default.
 * Other plans always store them (their next GEMMs read them): the call is
 * accepted there and changes nothing.  Like the timing probe, it changes the
 * plan and is not thread-safe.  MOE_ERR_NULL for a null plan;
 * MOE_ERR_UNSUPPORTED for keep = 1 on a fused-only plan (moe_config.mx_fused),
 * whose workspace has no room for the rows. */
moe_status moe_keep_intermediates(moe_plan plan, int keep);

/* Byte offset and size, inside the MX-fp8 saved-codes buffer
 * (moe_ffn_args.mx_saved), of the operands it holds, named and laid out as
 * the workspace's MX operands of moe_workspace_region (payload, or
 * "<name>.scales"): "mx_wdt", "mx_wgut", "mx_ht" and, with shared experts,
 * "mx_swdt", "mx_swgut", "mx_sht".  For tests and debugging.  MOE_ERR_NULL
 * for a null argument, MOE_ERR_INVALID for another name or a plan without
 * MX-fp8 experts (or shared experts, for the shared names). */
moe_status moe_mx_saved_region(moe_plan plan, const char* name, size_t* offset, size_t* bytes);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FFN_MI355X_H */
