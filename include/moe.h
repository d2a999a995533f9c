/*
 * moe.h - C ABI of the MI355X (gfx950) top-k MoE SwiGLU layer, forward pass.
 *
 * The layer (sources named by page title; section, equation or table):
 *   - router scores H = x.W_g, plus eps * Softplus(x.W_noise) when the noisy
 *     gate is on ("Llama 3 Meets MoE: Efficient Upcycling" review, section 3,
 *     noisy top-k router; "LLaMA-MoE v2" article, gating-mechanism section);
 *   - KeepTopK then softmax over the kept scores (Mixtral order), or softmax
 *     over all scores then top-k (ST order) (review, section 3 KeepTopK and
 *     G(x); section 5 router ablation);
 *   - per-expert capacity: assignments past an expert's capacity are dropped
 *     and add nothing to the output (review, section 3, capacity factor);
 *   - experts are SwiGLU FFNs down(SiLU(gate x) * up x) without bias
 *     (LLaMA-MoE v2 article, code example, class Expert);
 *   - y = s * sum_j G_j E_j(x) over the kept experts (review, section 3, MoE
 *     output; LLaMA-MoE v2 article, rescaling section, s = N/k).
 *
 * Conventions shared by every entry point
 *   Memory      Every tensor pointer is caller-owned DEVICE memory, row-major
 *               and contiguous; the library never allocates, frees or keeps
 *               device state. x, weights, x_perm, y_perm and y must be 16-byte
 *               aligned; ws must be 256-byte aligned and hold at least
 *               moe_workspace_bytes(cfg) bytes.
 *   Shapes      T tokens, H hidden, F per-expert intermediate, N experts,
 *               k experts per token. H % 8 == 0 is required (16-byte rows).
 *   Dtypes      act/wt = MOE_BF16/MOE_BF16 or MOE_F32/MOE_F32. Router weights
 *               (W_g, W_noise), eps, logits, gate weights, y_perm and the
 *               statistics are always fp32. y is cfg->out (fp32 or bf16).
 *   Streams     Every call is asynchronous on the given HIP stream; no call
 *               synchronises the host. Expert row counts stay on the device.
 *   Errors      Argument errors return before any launch (MOE_ERR_INVALID,
 *               MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE). A failed launch
 *               returns MOE_ERR_DEVICE. Faults inside kernels surface at the
 *               caller's next synchronisation. No C++ exception crosses the
 *               ABI. moe_last_error() gives a thread-local message.
 *   Outputs     Every output is fully overwritten (dropped tokens get y = 0).
 *               Pointers ending in _opt may be NULL.
 *   Determinism Results are bitwise reproducible for a fixed cfg and inputs:
 *               no floating-point atomics, fixed-order reductions.
 *   T == 0      Valid: per-expert outputs (counts, offsets, statistics) are
 *               zeroed; nothing else is touched.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,      /* bad argument: null pointer, k > N, T < 0, misalignment, ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented: H % 8 != 0, mixed act/wt dtypes, N > 64 */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes below moe_workspace_bytes(cfg) */
  MOE_ERR_DEVICE = 4        /* a HIP launch or runtime call failed */
} moe_status;

enum { MOE_F32 = 0, MOE_BF16 = 1 };                                    /* moe_dtype */
enum { MOE_TOPK_THEN_SOFTMAX = 0, MOE_SOFTMAX_THEN_TOPK = 1 };         /* moe_order */

typedef struct {
  int64_t T;            /* tokens, >= 0 */
  int32_t H;            /* hidden size, multiple of 8 */
  int32_t F;            /* per-expert intermediate size, >= 1 */
  int32_t N;            /* experts, 1..64 (config key num_local_experts) */
  int32_t k;            /* experts per token, 1..N (config key num_experts_per_tok) */
  int32_t capacity;     /* per-expert cap on kept assignments; < 0 = no cap (dropless) */
  int32_t order;        /* MOE_TOPK_THEN_SOFTMAX (Mixtral, default) or MOE_SOFTMAX_THEN_TOPK (ST) */
  int32_t noisy;        /* 1: add eps * Softplus(x.W_noise) to the router scores */
  int32_t want_stats;   /* 1: moe_route / moe_forward may fill load, importance, P, balance */
  float out_scale;      /* s: 1, or N/k for the rescaled LLaMA-MoE layer */
  int32_t act;          /* MOE_BF16 or MOE_F32: x, x_perm and the SwiGLU product h */
  int32_t wt;           /* expert weights; must equal act */
  int32_t out;          /* y: MOE_F32 or MOE_BF16 */
} moe_cfg;

/* Expert capacity = tokens per batch / N * CF, rounded up (review, section 3,
 * capacity-factor equation). count_assignments = 1 counts the T*k
 * (token, expert) assignments instead of the T tokens. Returns -1 for
 * cf < 0 or a result above INT32_MAX. Host only. */
int32_t moe_capacity(int64_t T, int32_t N, int32_t k, double cf, int32_t count_assignments);

/* Validates cfg on the host; never touches the device. Shapes are bounded so
 * that every operand is addressed with 32-bit byte offsets: T*H, T*k*F, T*k*H
 * and F*H below 2^29 elements, and for bf16 activations the router's partial
 * logits (T*N*(1+noisy) per 256-512-row chunk of H) below 2^29 floats;
 * beyond them it returns MOE_ERR_UNSUPPORTED. */
moe_status moe_check(const moe_cfg* cfg);

/* Workspace bytes that any entry point below needs for cfg (0 if cfg is
 * invalid). One workspace of this size serves every call with this cfg. */
size_t moe_workspace_bytes(const moe_cfg* cfg);

/* Router, KeepTopK and gate weights (review, section 3, H(x), KeepTopK, G(x);
 * section 5 for the ST order).
 *   x [T,H] act; Wg [H,N] fp32; Wn [H,N] fp32 and eps [T,N] fp32 (standard
 *   normal draws, one per token and expert) are read only when cfg->noisy.
 *   logits_opt [T,N] fp32: clean router logits x.W_g.
 *   topk_idx [T,k] int32: the k highest scores per token, in descending
 *   order, ties to the lower expert index. A NaN score (from NaN or Inf in x
 *   or the router weights) counts as -inf: it ranks below every number and
 *   adds 0 to the softmax denominators, so exactly k experts are kept.
 *   topk_w [T,k] fp32: Mixtral: softmax over the k kept scores; ST: softmax
 *   over all N scores taken at the kept experts (not renormalised).
 *   Statistics, written when cfg->want_stats and the pointer is non-NULL
 *   (LLaMA-MoE v2 article, gating section, balance loss; the LLaMA-MoE
 *   monitoring list names Gate Load and Gate Importance):
 *   load_opt [N] int32 assignments per expert before capacity;
 *   importance_opt [N] fp32 sum of gate weights per expert;
 *   P_opt [N] fp32 mean over tokens of softmax(logits);
 *   balance_opt [1] fp32 sum_i f_i P_i with f_i = load_i / (T k)
 *   (the coefficient lambda is left to the caller);
 *   smooth_load_opt [N] fp32, noisy gate only (MOE_ERR_INVALID otherwise):
 *   the smooth load estimate of the TopK Noisy Gate (Shazeer et al. 2017,
 *   which the LLaMA-MoE hub page names), sum over tokens of
 *   Phi(((x.W_g)_i - kth_excluding(H, k, i)) / Softplus((x.W_noise)_i)), the
 *   chance that expert i stays in the top k when only its own normal draw
 *   is taken again; kth_excluding is the k-th highest score of the other
 *   experts (-inf when k = N).
 *   ws: a workspace of moe_workspace_bytes(cfg) is required when statistics
 *   are requested or x is bf16 (the matrix-core router keeps its partial
 *   logits, one set per chunk of H, there); otherwise it may be NULL.
 *   Returns MOE_ERR_WORKSPACE when it is too small. */
moe_status moe_route(const moe_cfg* cfg, const void* x, const float* Wg, const float* Wn, const float* eps,
                     float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* load_opt,
                     float* importance_opt, float* P_opt, float* balance_opt, float* smooth_load_opt, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Capacity clip and permutation into expert-contiguous order (review,
 * section 3, capacity factor: each expert keeps its first cfg->capacity
 * assignments in token order; the rest are dropped).
 *   counts [N] int32 assignments per expert before capacity.
 *   offsets [N+1] int32 exclusive scan of kept = min(counts, capacity);
 *   offsets[N] = number of kept rows A.
 *   slot [T,k] int32 row of assignment (t,j), or -1 when dropped.
 *   row_token [T*k] int32 token of each row; -1 for rows >= A.
 *   x_perm [T*k,H] act (optional): rows gathered as x_perm[r] = x[row_token[r]];
 *   rows >= A are left untouched. NULL skips the gather (moe_grouped_swiglu
 *   can gather on the fly from x and row_token). */
moe_status moe_permute(const moe_cfg* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* row_token, void* x_perm, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU experts over the permuted rows (LLaMA-MoE v2 article, code
 * example, class Expert): for rows r in expert e's segment
 * [offsets[e], offsets[e+1]):
 *   h[r]      = SiLU(a_r . Wgate[e]^T) * (a_r . Wup[e]^T), rounded to act
 *   y_perm[r] = h[r] . Wdown[e]^T                              (fp32)
 * with a_r = x_perm_or_x[r] when row_token_opt is NULL, else
 * a_r = x_perm_or_x[row_token_opt[r]] (gather fused into the loads).
 *   Wgate, Wup [N,F,H] wt; Wdown [N,H,F] wt; y_perm [T*k,H] fp32, rows >= A
 *   untouched. The intermediate h lives in ws. */
moe_status moe_grouped_swiglu(const moe_cfg* cfg, const void* x_perm_or_x, const int32_t* row_token_opt,
                              const int32_t* offsets, const void* Wgate, const void* Wup, const void* Wdown,
                              float* y_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Gate-weighted combine back to token order (review, section 3, MoE output;
 * LLaMA-MoE v2 article, rescaling section):
 *   y[t] = s * sum_{j=0..k-1, slot[t,j] >= 0} topk_w[t,j] * y_perm[slot[t,j]]
 * summed in j order in fp32; a token with every slot dropped gets y = 0.
 *   y_perm [T*k,H] fp32; a slot at or past T*k counts as dropped.
 *   y [T,H] cfg->out. Needs no workspace. */
moe_status moe_combine(const moe_cfg* cfg, const float* y_perm, const int32_t* slot, const float* topk_w,
                       void* y, hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_swiglu (gather fused)
 * and moe_combine on one stream without host synchronisation. Optional
 * outputs: topk_idx_opt [T,k], topk_w_opt [T,k], kept_opt [N] (after
 * capacity), load_opt [N] (before capacity), and the statistics as in
 * moe_route.
 *   Device-side failure: in the persistent expert kernel (bf16 prefill
 *   shapes) a down-projection tile waits, with a bounded number of polls, for
 *   the gate/up tiles of its rows. If a wait ever gives up, that tile writes
 *   NaN over its y_perm rows and the combine writes every element of y as
 *   NaN, so the failure cannot pass as a result (moe_grouped_swiglu alone
 *   leaves the NaN rows in y_perm). The call still returns MOE_OK, since no
 *   call synchronises the host. */
moe_status moe_forward(const moe_cfg* cfg, const void* x, const float* Wg, const float* Wn, const float* eps,
                       const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* topk_idx_opt,
                       float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt, float* importance_opt,
                       float* P_opt, float* balance_opt, float* smooth_load_opt, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* The residual (shared-neuron, "Inter" mode) layer: an always-active shared
 * slice of F_shared SwiGLU neurons added to the routed experts (LLaMA-MoE
 * hub page, shared-neuron partitioning, Inter mode; LLaMA-MoE v2 article,
 * shared-neuron partitioning):
 *   y[t] = FFN_shared(x[t]) + s * sum_{kept j} topk_w[t,j] * E_{idx[t,j]}(x[t])
 * FFN_shared(x) = Ws_down . (SiLU(Ws_gate . x) * (Ws_up . x)), h rounded to
 * act as in the experts; the rescale s applies to the routed sum only.
 *   Ws_gate, Ws_up [F_shared,H] wt; Ws_down [H,F_shared] wt, 16-byte aligned.
 *   Everything else as moe_forward. The workspace must hold
 *   moe_residual_workspace_bytes(cfg, F_shared) bytes (0 if invalid).
 *   The shared slice runs as a one-expert layer over all T rows through the
 *   same expert kernels, then the routed layer; the combine adds the two. */
size_t moe_residual_workspace_bytes(const moe_cfg* cfg, int32_t F_shared);
moe_status moe_forward_residual(const moe_cfg* cfg, int32_t F_shared, const void* x, const float* Wg, const float* Wn,
                                const float* eps, const void* Wgate, const void* Wup, const void* Wdown,
                                const void* Ws_gate, const void* Ws_up, const void* Ws_down, void* y,
                                int32_t* topk_idx_opt, float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt,
                                float* importance_opt, float* P_opt, float* balance_opt, float* smooth_load_opt,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Training: a forward that keeps what the backward needs, and the backward
 * of the layer (continual pre-training is the pages' main workload:
 * LLaMA-MoE hub page and paper summary, continual pre-training; the balance
 * loss is the LLaMA-MoE v2 article's gating section).
 *   Shapes: bf16 activations and weights, F % 8 == 0, more than 48 rows per
 *   expert on average (the persistent expert kernel's shapes); otherwise
 *   MOE_ERR_UNSUPPORTED. ws holds moe_train_workspace_bytes(cfg) bytes.
 *   moe_forward_train computes the same layer as moe_forward (same bits of
 *   y and the statistics) and leaves in ws the routing, the router logits,
 *   the gate/up pre-activations g and u (fp32), h and the expert outputs.
 *   moe_backward must follow it on the same stream with the same cfg, inputs
 *   and ws, untouched in between. It returns the gradients of
 *   L = <dy, y> + d_balance * balance:
 *     dy [T,H] fp32; dx [T,H] fp32; dWg [H,N] fp32; dWn_opt [H,N] fp32
 *     (required when noisy); dWgate, dWup [N,F,H] fp32; dWdown [N,H,F] fp32.
 *   KeepTopK and the capacity clip are piecewise constant: the router gets
 *   gradient only through the chosen experts' gate weights (Mixtral: softmax
 *   over the kept scores; ST: softmax over all), a dropped slot gets none,
 *   and f_i of the balance is a count (no gradient); the noise path
 *   differentiates Softplus to the sigmoid. Matrix-core operands are bf16
 *   (dE = s w dy and the SwiGLU gradients dg, du, rounded to nearest even),
 *   every sum is fp32. Results are bitwise reproducible. */
size_t moe_train_workspace_bytes(const moe_cfg* cfg);
moe_status moe_forward_train(const moe_cfg* cfg, const void* x, const float* Wg, const float* Wn, const float* eps,
                             const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* kept_opt,
                             int32_t* load_opt, float* importance_opt, float* P_opt, float* balance_opt,
                             float* smooth_load_opt, void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_backward(const moe_cfg* cfg, const void* x, const float* Wg, const float* Wn, const float* eps,
                        const void* Wgate, const void* Wup, const void* Wdown, const float* dy, float d_balance,
                        float* dx, float* dWg, float* dWn_opt, float* dWgate, float* dWup, float* dWdown, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, outputs and results as
 * moe_forward, minus ws and ws_bytes; it allocates nothing and makes no
 * allocating call.
 *   The workspace is a static device array of moe_noalloc_scratch_bytes()
 *   bytes (320 MiB) that each GPU the library runs on holds until the
 *   process ends; its device address is looked up on a device's first call.
 *   It covers the LLaMA-MoE-3.5B layers (4096 tokens: 2/8 needs 157 MB, 4/16
 *   with top-4 291 MB); a layer whose moe_workspace_bytes(cfg) exceeds it is
 *   rejected with MOE_ERR_WORKSPACE before any launch.
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind; each call re-initialises what it needs (the expert kernel's queue
 *   counters are cleared on the stream). Calls that overlap on one GPU (on
 *   different streams, or from several threads without ordering) race on the
 *   array and give undefined results. */
moe_status moe_forward_noalloc(const moe_cfg* cfg, const void* x, const float* Wg, const float* Wn, const float* eps,
                               const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* topk_idx_opt,
                               float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt, float* importance_opt,
                               float* P_opt, float* balance_opt, float* smooth_load_opt, hipStream_t stream);
size_t moe_noalloc_scratch_bytes(void);

const char* moe_status_str(moe_status s);
const char* moe_last_error(void); /* thread-local text of the last failure, "" if none */

/* Kernel timing for benchmarks. moe_profile_select(id) makes the library
 * bracket every later launch of kernel `id` (MOE_KERNEL_*) with a pair of HIP
 * events on the launch stream; -1 turns it off. The first call with id >= 0
 * creates a pool of 4096 event pairs (the only HIP objects the library
 * creates; they live until the process ends), so a timed launch costs two
 * hipEventRecord calls; launches past the pool's size before the next read
 * are not timed. moe_profile_read() waits for the recorded events, returns
 * the summed duration in ms and the number of launches timed, and clears the
 * record. Host only. */
enum {
  MOE_KERNEL_ROUTER = 0,
  MOE_KERNEL_HIST = 1,
  MOE_KERNEL_SCATTER = 2,
  MOE_KERNEL_GATHER = 3,
  MOE_KERNEL_GEMM1 = 4,
  MOE_KERNEL_GEMM2 = 5,
  MOE_KERNEL_COMBINE = 6,
  MOE_KERNEL_STATS = 7,
  MOE_KERNEL_EXPERTS = 8,  /* both expert GEMMs in one persistent launch (bf16, prefill shapes) */
  MOE_KERNEL_BWD_GATE = 9,       /* backward: gate weights to the router, dE */
  MOE_KERNEL_BWD_DGRAD = 10,     /* backward: dh with the SwiGLU derivative, dx of the experts, and dWdown */
  MOE_KERNEL_BWD_DX = 11,        /* backward: dx gathered back to tokens, with the router terms */
  MOE_KERNEL_BWD_WGRAD = 12,     /* backward: the weight gradients dWgate and dWup */
  MOE_KERNEL_BWD_ROUTER = 13,    /* backward: router and noise weight gradients */
  MOE_KERNEL_COUNT = 14
};
moe_status moe_profile_select(int32_t kernel_id);
moe_status moe_profile_read(double* total_ms, int64_t* launches);

/* Test hook for the expert kernel's bounded wait (see moe_forward). Later
 * launches poll at most spin_limit times (<= 0: the default, about a second)
 * and wait for wait_extra more finished gate/up tiles than exist, so with
 * wait_extra > 0 every wait gives up after spin_limit polls and the failure
 * path runs while every kernel still ends normally. moe_debug_set_wait(0, 0)
 * restores normal operation. Process-wide, host only; MOE_ERR_INVALID for
 * wait_extra < 0. */
moe_status moe_debug_set_wait(int32_t spin_limit, int32_t wait_extra);

/* Bounds checks. Every index that data can steer (a slot, a row_token entry,
 * the offsets) is guarded in every build: an out-of-range value is dropped or
 * clamped, never followed. The debug build, libmoe_debug.so (compiled with
 * -DMOE_DEBUG; moe_debug_build() returns 1 there, 0 in libmoe.so), also
 * records each guard that fires by setting a bit of a 32-bit word in the
 * workspace at byte offset moe_debug_word_offset(cfg) (0 for an invalid
 * cfg; the same offset in the residual and training workspaces):
 *   1 a kept slot's row at or past T*k (scatter), 2 a row_token entry
 *   outside x (moe_permute's gather), 4 a slot past y_perm (combine),
 *   8 offsets outside [0, rows] or decreasing (expert GEMMs), 16 a slot past
 *   the rows in the backward.
 * The library never clears the word; the caller zeroes it. On valid input no
 * bit is set. The release build never writes it. For tests and debugging;
 * the debug build is as fast as the release build up to the atomics of
 * guards that fire. */
int32_t moe_debug_build(void);
size_t moe_debug_word_offset(const moe_cfg* cfg);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
