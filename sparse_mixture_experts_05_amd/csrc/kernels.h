// Launch interface between the host ABI layer (moe_abi.cpp) and the kernels.
// Every launcher enqueues on the given stream and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router + KeepTopK + gates (router.hip) --------------------------------
struct RouterParams {
  const void* x;          // [T,H] act
  int act_bf16;
  const float* Wg;        // [H,N]
  const float* Wn;        // [H,N] (noisy)
  const float* eps;       // [T,N] (noisy)
  int64_t T;
  int H, N, k, order, noisy;
  float* logits;          // [T,N] or null
  float* noise_logits;    // [T,N] x.W_noise (noisy), or null
  int32_t* topk_idx;      // [T,k]
  float* topk_w;          // [T,k]
  int32_t* hist;          // [blocks,N] assignments per expert per block, or null
  float* stat_part;       // [blocks,3N] importance, sum of softmax(logits), smooth load; or null
  int smooth;             // 1: fill the smooth-load partials (noisy gate only)
  float* part;            // bf16 x: router_part_floats(T, H, N, noisy) fp32 of workspace, the
                          // per-chunk partial logits
};
constexpr int kStatsPerExpert = 3;  // importance, softmax(logits) sum, smooth load
// Tokens handled by one router block; the permutation scatter reads the
// per-block histogram with this granularity.
int router_tokens_per_block(int N, int noisy, int act_bf16);
int router_blocks(int64_t T, int N, int noisy, int act_bf16);
hipError_t launch_router(const RouterParams& p, hipStream_t s);
hipError_t launch_router_mma(const RouterParams& p, hipStream_t s);
// Floats of the matrix-core router's partial logits (one set per chunk of H).
int64_t router_part_floats(int64_t T, int H, int N, int noisy);

// Fixed-order reduction of the router's per-block statistics.
struct StatsParams {
  const int32_t* hist;
  const float* stat_part;
  int blocks;
  int64_t T;
  int N, k;
  int32_t* load;          // [N] or null
  float* importance;      // [N] or null
  float* P;               // [N] or null
  float* balance;         // [1] or null
  float* smooth_load;     // [N] or null (needs the router's smooth partials)
};
hipError_t launch_stats(const StatsParams& p, hipStream_t s);

// Zero per-expert outputs (used for T == 0).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

// ---- permutation (permute.hip) ---------------------------------------------
// Histogram of a given topk_idx with the router's block granularity.
struct HistParams {
  const int32_t* topk_idx;
  int64_t T;
  int N, k, tokens_per_block;
  int32_t* hist;
};
hipError_t launch_hist(const HistParams& p, hipStream_t s);

struct ScatterParams {
  const int32_t* topk_idx;  // [T,k]
  const int32_t* hist;      // [ceil(T/hist_tokens), N]
  int hist_tokens;
  int64_t T;
  int N, k;
  int capacity;             // < 0: none
  int32_t* counts;          // [N] before capacity, or null
  int32_t* kept;            // [N] after capacity, or null
  int32_t* offsets;         // [N+1]
  int32_t* slot;            // [T,k]
  int32_t* row_token;       // [T*k]
  int32_t* zero;            // [zero_n] set to 0 by block 0 (the expert kernel's queue counters), or null
  int zero_n;
  int32_t* dbg;             // debug word, or null
};
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);

struct GatherParams {
  const void* x;
  void* x_perm;
  const int32_t* row_token;
  const int32_t* offsets;
  int64_t rows_max;       // T*k
  int H, N, elem_bytes;
  int64_t T;              // rows of x
  int32_t* dbg;           // debug word, or null
};
hipError_t launch_gather(const GatherParams& p, hipStream_t s);

// ---- grouped GEMMs (gemm_mfma.hip, gemm_simple.hip) -------------------------
// Rows of expert e are [offsets[e], offsets[e+1]). For each row r:
//   swiglu: C[r, f] = round(SiLU(a_r . B0[e,f,:]) * (a_r . B1[e,f,:]))   f < Nout
//   plain : C[split][r, n] = sum over this split's K range of a_r . B0[e,n,:]
// with a_r = A[row_token[r]] when row_token is set, else A[r].
struct GemmParams {
  const void* A;
  int64_t lda;
  const int32_t* row_token;   // gather, or null
  const int32_t* offsets;     // [N+1]
  int N;                      // experts
  const void* B0;
  const void* B1;             // swiglu only
  int64_t b_expert_stride;    // elements between experts in B0/B1
  int64_t ldb;                // = K
  int K;
  int Nout;                   // output columns (F for swiglu, H for plain)
  void* C;
  int64_t ldc;
  int64_t c_split_stride;     // elements between split-K partial outputs
  int splits;
  int64_t rows_max;           // upper bound on offsets[N] (grid sizing)
  int64_t a_rows;             // rows of A (bounds of the gathered or permuted operand)
  int swiglu;
  // training: the swiglu epilogue also stores g and u (fp32) as
  // gu[r, f] and gu[r, Nout + f] (row stride 2*Nout), when gu is set
  float* gu;
  // 1: the SwiGLU backward epilogue of a plain GEMM whose sum is dh[r, f]:
  // with g, u from gu, C[r, f] = bf16(dh u SiLU'(g)) and
  // C[r, Nout + f] = bf16(dh SiLU(g)) (C row stride ldc = 2*Nout)
  int epi;
  // the backward's K-outer ("KN") B operand: row k of the K range is row k of
  // B0 when k < ksplit, else row k - ksplit of B1 (each b_rows rows of ldb
  // elements per expert); the N columns are contiguous within a row
  int64_t b_rows;
  int ksplit;
  int32_t* dbg;               // debug word, or null
};
// Decode-shaped tiles (few rows per expert), one launch per GEMM.
hipError_t launch_gemm_decode(const GemmParams& p, hipStream_t s);
bool gemm_bf16_mfma_supported(int K, int Nout);
bool gemm_decode_shape(int64_t rows_max, int N);
void gemm_decode_tile(int* bm, int* bn);
hipError_t launch_gemm_simple(const GemmParams& p, int bf16, hipStream_t s);

// The backward's weight gradients on the same 256 x 256 tile, one tile per
// workgroup: per expert e, K over the expert's rows r in [offsets[e],
// offsets[e+1]) of the permuted order, C_e[m][n] = sum_r A[r][m] B[r'][n] into
// the e-th [M, Nout] block of C (c_split_stride = M * Nout). Both operands are
// K-outer: A rows of lda elements (a_rows of them), the M columns contiguous;
// B rows of ldb elements (b_rows of them), r' = row_token[r] when row_token is
// set, else r. With C2 set, the same launch also runs a second gradient of
// the same shape whose A columns start a2_col elements further along each
// row and whose output is C2 (its m-tiles follow the first one's).
struct WgradParams {
  GemmParams g;
  int M;
  void* C2;
  int64_t a2_col;
};
hipError_t launch_gemm_wgrad(const WgradParams& wp, hipStream_t s);

// Both expert GEMMs in one persistent launch: g1 is the gate/up GEMM with the
// SwiGLU epilogue (writing h), g2 the down projection reading h (no K split).
// sched: fused_sched_ints(rows_max, N) int32 of workspace, zero on entry.
// A down tile waits for its row block's gate/up tiles at most spin_limit
// polls; if it gives up it raises sched[fused_error_index()] and writes NaN
// over its outputs. wait_extra raises the awaited count (0 in use; a test
// sets it so that every wait gives up).
struct FusedParams {
  GemmParams g1, g2;
  int32_t* sched;
  StatsParams st;  // router statistics, reduced once the queue is empty
  int stats;       // 1: reduce them (in the workgroup that draws the first ticket past the end)
  int spin_limit;
  int wait_extra;
  // the backward only: a third GEMM whose tiles never wait (the weight
  // gradient dWdown, laid out as for launch_gemm_wgrad with M = m3), run from
  // the same queue to fill the compute units the dependent tiles leave idle;
  // none when g3.N == 0
  GemmParams g3;
  int m3;
};
constexpr int kDefaultSpinLimit = 1 << 22;  // about a second of polling
int fused_error_index();
int fused_sched_ints(int64_t rows_max, int N);
bool gemm_fused_supported(int64_t rows_max, int N, int K1, int F);
hipError_t launch_experts_fused(const FusedParams& fp, hipStream_t s);
// The backward's input gradients in the same persistent kernel: g1 = dh with
// the SwiGLU-derivative epilogue (epi 1, writing dg|du), g2 = dx reading
// dg|du, both with the weights as K-outer B operands; g3 (dWdown) fills the
// queue's idle units.
hipError_t launch_bwd_dgrad_fused(const FusedParams& fp, hipStream_t s);

// ---- combine (combine.hip) --------------------------------------------------
struct CombineParams {
  const float* y_perm;       // [splits][rows][H]
  int64_t split_stride;      // elements
  int splits;
  const int32_t* slot;       // [T,k]
  const float* topk_w;       // [T,k]
  void* y;                   // [T,H]
  int out_bf16;
  int64_t T;
  int H, k;
  float scale;
  const int32_t* error;      // *error != 0: an earlier kernel failed, and y is written as all NaN. May be null.
  const float* residual;     // [res_splits][T][H]: added unscaled, y = residual + s * sum; or null
  int64_t res_split_stride;  // elements
  int res_splits;
  int64_t rows;              // rows of y_perm (per split); a slot at or past it adds nothing
  int32_t* dbg;              // debug word, or null
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

// ---- backward (backward.hip) -------------------------------------------------
struct BwdGateParams {
  int64_t T;
  int H, N, k, order, noisy;
  float scale;              // s
  float d_balance;          // upstream gradient of the balance statistic
  const float* dy;          // [T,H]
  const float* y_perm;      // [rows][H] expert outputs of the forward
  const int32_t* slot;      // [T,k]
  const int32_t* topk_idx;  // [T,k]
  const float* topk_w;      // [T,k]
  const float* logits;      // [T,N] clean logits of the forward
  const float* noise_logits;  // [T,N] (noisy)
  const float* eps;         // [T,N] (noisy)
  const int32_t* counts;    // [N] assignments before capacity
  uint16_t* dE;             // [rows][H] bf16: s w dy at each kept slot's row
  float* dlog;              // [T,N] gradient of the clean logits
  float* dnz;               // [T,N] gradient of the noise logits (noisy)
  int64_t rows;             // rows of y_perm and dE; a slot at or past it is skipped
  int32_t* dbg;             // debug word, or null
  int32_t* zero;            // zero_n int32 that block 0 sets to 0 (the next launch's queue), or null
  int zero_n;
};
hipError_t launch_bwd_gate(const BwdGateParams& p, hipStream_t s);

struct BwdDxParams {
  int64_t T;
  int H, N, k, noisy;
  const float* dx_perm;     // [rows][H]
  int64_t rows;             // rows of dx_perm
  const int32_t* slot;      // [T,k]
  const float* dlog;        // [T,N]
  const float* dnz;         // [T,N]
  const float* Wg;          // [H,N]
  const float* Wn;          // [H,N]
  float* dx;                // [T,H]
  int32_t* dbg;             // debug word, or null
};
hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s);

struct RouterWgradParams {
  int64_t T;
  int H, N, noisy;
  const uint16_t* x;        // [T,H] bf16
  const float* dlog;        // [T,N]
  const float* dnz;         // [T,N]
  float* part;              // [router_wgrad_chunks(T)][N * (1 + noisy)][H]
  float* dWg;               // [H,N]
  float* dWn;               // [H,N]
};
int router_wgrad_chunks(int64_t T);
hipError_t launch_router_wgrad(const RouterWgradParams& p, hipStream_t s);


}  // namespace moe
