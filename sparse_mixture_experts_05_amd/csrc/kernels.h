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
  int32_t* topk_idx;      // [T,k]
  float* topk_w;          // [T,k]
  int32_t* hist;          // [blocks,N] assignments per expert per block, or null
  float* stat_part;       // [blocks,2N] importance and sum of softmax(logits), or null
};
// Tokens handled by one router block; the permutation scatter reads the
// per-block histogram with this granularity.
int router_tokens_per_block(int N, int noisy, int act_bf16);
int router_blocks(int64_t T, int N, int noisy, int act_bf16);
hipError_t launch_router(const RouterParams& p, hipStream_t s);
hipError_t launch_router_mma(const RouterParams& p, hipStream_t s);

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
};
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);

struct GatherParams {
  const void* x;
  void* x_perm;
  const int32_t* row_token;
  const int32_t* offsets;
  int64_t rows_max;       // T*k
  int H, N, elem_bytes;
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
};
hipError_t launch_gemm_bf16_mfma(const GemmParams& p, hipStream_t s);
bool gemm_bf16_mfma_supported(int K, int Nout);
void gemm_bf16_mfma_tile(int64_t rows_max, int N, int* bm, int* bn);
hipError_t launch_gemm_simple(const GemmParams& p, int bf16, hipStream_t s);

// Both expert GEMMs in one persistent launch: g1 is the gate/up GEMM with the
// SwiGLU epilogue (writing h), g2 the down projection reading h (no K split).
// sched: fused_sched_ints(rows_max, N) int32 of workspace, zero on entry.
struct FusedParams {
  GemmParams g1, g2;
  int32_t* sched;
  StatsParams st;  // router statistics, reduced once the queue is empty
  int stats;       // 1: reduce them (in the workgroup that draws the first ticket past the end)
};
int fused_sched_ints(int64_t rows_max, int N);
bool gemm_fused_supported(int64_t rows_max, int N, int K1, int F);
hipError_t launch_experts_fused(const FusedParams& fp, hipStream_t s);

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
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s);

}  // namespace moe
