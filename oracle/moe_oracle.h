/*
 * CPU ORACLE for the top-k MoE SwiGLU layer: the forward pass, the
 * shared-neuron (residual) layer, the smooth gate load, and the backward.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow, obviously-correct
 * reference the GPU path is checked against. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product library
 * never links, calls or falls back to it.
 *
 * All arithmetic is IEEE double unless a rounding step is stated. Inputs are
 * the exact values the GPU sees (fp32 arrays, or bf16 bit patterns decoded
 * exactly). Outputs are plain host arrays. No blocking, fusion or reordering
 * beyond what each definition states.
 *
 * Sources (page titles as printed on the pages):
 *   [UP]  "Llama 3 Meets MoE: Efficient Upcycling" (paper review), section 3
 *         core formulas: MoE output y = sum_i G(x)_i E_i(x); noisy top-k
 *         router G = Softmax(KeepTopK(H, k)) with
 *         H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i);
 *         KeepTopK; expert capacity = tokens per batch / N * CF with
 *         overflow tokens skipping the experts; section 5 router ablation
 *         (Mixtral order vs ST order).
 *   [V2]  "LLaMA-MoE v2" article: gating-mechanism section (noisy gate,
 *         balance loss L = lambda * sum f_i P_i), rescaling section
 *         (y = N/k * sum G_i E_i), and its code example (SwiGLU expert
 *         down(SiLU(gate x) * up x), noise = randn * softplus(noise_linear)),
 *         and its shared-neuron partitioning (an always-active slice).
 *   [HUB] LLaMA-MoE hub page: the expert-construction list (Inter / Inner
 *         shared neurons), the gate choices (TopK Noisy Gate; Switch) and the
 *         Gate Load monitor, and continual pre-training (the backward).
 *   The smooth gate load follows the noisy top-k gate's original paper
 *   (Shazeer et al. 2017), which the hub page names.
 *
 * Parity status: every function here is pinned by CPU tests (brute force on
 * tiny inputs, closed forms, library routines, invariants); none is
 * "parity unpinned".
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };                 /* storage of x / expert weights */
enum { ORC_H_EXACT = 0, ORC_H_F32 = 1, ORC_H_BF16 = 2 }; /* rounding of the SwiGLU product h */
enum { ORC_KEEPTOPK_SOFTMAX = 0, ORC_SOFTMAX_TOPK = 1 };

typedef struct {
  int64_t T;          /* tokens */
  int32_t H;          /* hidden size */
  int32_t F;          /* per-expert intermediate size */
  int32_t N;          /* experts */
  int32_t k;          /* experts per token */
  int64_t capacity;   /* per-expert cap on kept assignments; < 0 means no cap */
  int32_t order;      /* ORC_KEEPTOPK_SOFTMAX (Mixtral) or ORC_SOFTMAX_TOPK (ST) */
  int32_t noisy;      /* add eps * softplus(x W_noise) to the logits */
  double out_scale;   /* s in y = s * sum_j w_j E_j  (1, or N/k) */
  int32_t h_round;    /* ORC_H_* */
  int32_t x_dtype;    /* ORC_F32 / ORC_BF16 */
  int32_t w_dtype;    /* ORC_F32 / ORC_BF16 (expert weights) */
} oracle_cfg;

/* Router + KeepTopK + gate weights for every token.
 * x [T,H] (x_dtype), Wg [H,N] fp32, Wn [H,N] fp32 and eps [T,N] fp32 (used iff noisy).
 * Out: logits [T,N] fp32 = fl32(x.Wg) (clean), Hv [T,N] fp32 = selection scores,
 *      topk_idx [T,k] (sorted by Hv descending, ties to the lower index;
 *      a NaN score is stored and ranked as -inf),
 *      topk_w [T,k] double, min_gap [T] double (smallest gap between adjacent
 *      sorted scores among the first min(k+1, N); +inf when N == 1). */
int oracle_route(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                 float* logits, float* Hv, int32_t* topk_idx, double* topk_w, double* min_gap);

/* Gate load / importance / balance statistics (before capacity).
 * load[N], importance[N], P[N], f[N]; balance = sum f_i P_i;
 * balance_code = the article's code variant (gate-weighted frequency with a
 * 1e-6 guard, times N), reported for information only. */
int oracle_stats(const oracle_cfg* c, const float* logits, const int32_t* topk_idx, const double* topk_w,
                 int64_t* load, double* importance, double* P, double* f, double* balance,
                 double* balance_code);

/* Smooth gate load of the noisy top-k gate (the TopK Noisy Gate of Shazeer et
 * al. 2017 that the LLaMA-MoE hub page names, with its Gate Load monitor):
 *   smooth_load_i = sum_t P(x_t, i),
 *   P(x, i) = Phi( (fl32((x.W_g)_i) - kth_excluding(H(x), k, i)) / Softplus((x.W_noise)_i) ),
 * the probability that expert i is among the top k when only its own normal
 * draw is taken again. kth_excluding(H, k, i) is the k-th highest of the
 * other experts' scores H (fp32, as oracle_route stores them), or -inf when
 * fewer than k others exist; Phi is the standard normal CDF. Needs noisy. */
int oracle_smooth_load(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                       double* smooth_load);

/* Capacity clip and expert-contiguous permutation.
 * counts[N] (before capacity), kept[N] = min(counts, C), offsets[N+1] =
 * exclusive scan of kept, slot[T,k] = row of (t,j) or -1 when dropped,
 * row_token[T*k] = token of each row, -1 past the last kept row. */
int oracle_capacity(const oracle_cfg* c, const int32_t* topk_idx, int64_t* counts, int64_t* kept,
                    int64_t* offsets, int64_t* slot, int64_t* row_token);

/* One expert applied to selected tokens: h_out [n,F] (after rounding, may be
 * NULL) and E_out [n,H] = down(round(SiLU(gate x) * up x)). */
int oracle_expert_rows(const oracle_cfg* c, const void* x, const void* Wgate, const void* Wup,
                       const void* Wdown, int32_t e, const int64_t* tokens, int64_t n, int32_t nthreads,
                       double* h_out, double* E_out);

/* Layer output for selected tokens, given routing and slots:
 * y_t = s * sum_{j=0..k-1, slot>=0} w_j E_{idx_j}(x_t), summed in j order.
 * y64 [n,H] double (may be NULL), y32 [n,H] = fl32(y64) (may be NULL). */
int oracle_combine_tokens(const oracle_cfg* c, const void* x, const void* Wgate, const void* Wup,
                          const void* Wdown, const int32_t* topk_idx, const double* topk_w,
                          const int64_t* slot, const int64_t* tokens, int64_t n, int32_t nthreads,
                          double* y64, float* y32);

/* The same combine as oracle_combine_tokens, from expert outputs computed
 * beforehand: E [n,k,H] holds E_{idx_j}(x_t) for the listed tokens (row j of
 * token i; rows of dropped slots are not read). One expert pass then serves
 * several capacity settings of the same routing.
 * y64 [n,H] double (may be NULL), y32 [n,H] = fl32(y64) (may be NULL). */
int oracle_combine_rows(const oracle_cfg* c, const double* topk_w, const int64_t* slot, const int64_t* tokens,
                        int64_t n, const double* E, double* y64, float* y32);

/* The residual (shared-neuron, "Inter" mode) layer of the LLaMA-MoE hub
 * page's construction list and the LLaMA-MoE v2 article's shared-neuron
 * section: a slice of always-active neurons R(x) = FFN_shared(x) added to the
 * routed experts,  y_t = R(x_t) + s * sum_j w_j E_{idx_j}(x_t)  (kept j, in
 * j order). R [n,H] holds R(x_t) of the listed tokens (oracle_expert_rows of
 * the shared slice as a one-expert layer); E [n,k,H] as in
 * oracle_combine_rows. */
int oracle_residual_combine_rows(const oracle_cfg* c, const double* topk_w, const int64_t* slot,
                                 const int64_t* tokens, int64_t n, const double* E, const double* R, double* y64,
                                 float* y32);

/* Backward of the layer, for a training step (continual pre-training is the
 * pages' main workload: LLaMA-MoE hub page and paper summary, continual
 * pre-training; the balance loss of the LLaMA-MoE v2 article's gating
 * section). Given the upstream gradient dy [T,H] of the layer output and
 * d_balance, the upstream gradient of the balance statistic sum_i f_i P_i
 * (lambda of the article; f_i is a count and carries no gradient), it
 * returns the gradients of L = <dy, y> + d_balance * balance:
 *   dx [T,H], dWg [H,N], dWn [H,N] (zeroed unless noisy),
 *   dWgate, dWup [N,F,H], dWdown [N,H,F]   (all double).
 * Routing (KeepTopK and the capacity clip) is piecewise constant: no
 * gradient flows through the choice of experts or slots, only through the
 * gate weights of the chosen ones. The forward is recomputed here in the
 * same way as the oracle's forward (h rounded per h_round). With
 * h_round = ORC_H_BF16 the backward rounds to bf16 where the bf16 layer
 * feeds matrix cores: the expert-output gradient dE = s w dy and the SwiGLU
 * gradients dg, du; otherwise nothing is rounded (exact mode, for finite
 * differences). nthreads spreads the experts, then the tokens, then the rows of
 * dWg over threads; every sum keeps a fixed order (an expert's rows in token
 * order, a token's slots in slot order, the tokens in order), so the result
 * does not depend on the thread count. */
int oracle_backward(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                    const void* Wgate, const void* Wup, const void* Wdown, const float* dy, double d_balance,
                    int32_t nthreads, double* dx, double* dWg, double* dWn, double* dWgate, double* dWup,
                    double* dWdown);

/* Scalar pieces, exported so tests can pin them against library routines. */
double oracle_round_bf16(double v);   /* round to nearest bf16, ties to even */
double oracle_round_f32(double v);    /* round to nearest fp32, ties to even */
double oracle_silu(double z);
double oracle_softplus(double z);

#ifdef __cplusplus
}
#endif
#endif
