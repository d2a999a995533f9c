// Grouped GEMMs of the SwiGLU experts on the vector ALUs, for shapes the
// matrix-core kernel does not take: fp32 activations and weights, or an
// intermediate size F that is not a multiple of 8. Same row grouping and
// device-side tile lookup as the matrix-core kernel; element-wise loads, so
// any F and any alignment of F-long rows is accepted.
//
// Tile: 64 rows x 64 output columns, K in steps of 16 through LDS; each of
// the 256 threads accumulates a 4 x 4 block in fp32 (gate and up blocks for
// the SwiGLU form, LLaMA-MoE v2 article, code example, class Expert).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int TM = 64, TN = 64, TK = 16;

template <typename T, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void k_gemm_simple(GemmParams p) {
  __shared__ float sA[TK][TM + 1];
  __shared__ float sB0[TK][TN + 1];
  __shared__ float sB1[SWIGLU ? TK : 1][TN + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int ntiles = (p.Nout + TN - 1) / TN;
  const int mtiles = static_cast<int>((p.rows_max + TM - 1) / TM) + p.N;
  int bid = blockIdx.x;
  const int nt = bid % ntiles;
  bid /= ntiles;
  const int mt = bid % mtiles;
  const int split = bid / mtiles;
  TileInfo ti;
  if (!find_tile<TM>(p.offsets, p.N, static_cast<int>(p.rows_max), mt, ti, p.dbg)) return;

  const int kper = (p.K + p.splits - 1) / p.splits;
  const int kb0 = split * kper;
  const int kb1 = min(p.K, kb0 + kper);

  const T* __restrict__ A = static_cast<const T*>(p.A);
  const T* __restrict__ B0 = static_cast<const T*>(p.B0) + ti.expert * p.b_expert_stride;
  const T* __restrict__ B1 = SWIGLU ? static_cast<const T*>(p.B1) + ti.expert * p.b_expert_stride : nullptr;

  // each thread loads 4 elements of each tile per K step: row/col = e / TK, k = e % TK
  int64_t arow[4];
  bool aval[4];
  int64_t bcol[4];
  bool bval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + i * 256;
    const int r = e / TK;
    aval[i] = r < ti.rows;
    int64_t src = ti.row0 + r;
    if (GATHER) {
      src = aval[i] ? p.row_token[src] : 0;
      aval[i] = aval[i] && src >= 0 && src < p.a_rows;  // a row_token entry outside x reads zeros
    }
    arow[i] = aval[i] ? src * p.lda : 0;
    const int f = nt * TN + r;
    bval[i] = f < p.Nout;
    bcol[i] = bval[i] ? static_cast<int64_t>(f) * p.ldb : 0;
  }

  float acc0[4][4], acc1[SWIGLU ? 4 : 1][SWIGLU ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc0[i][j] = 0.0f;
  if constexpr (SWIGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc1[i][j] = 0.0f;
  }

  for (int k0 = kb0; k0 < kb1; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      const int r = e / TK, kk = e % TK;
      const bool kin = k0 + kk < kb1;
      sA[kk][r] = (aval[i] && kin) ? Elem<T>::load(A, arow[i] + k0 + kk) : 0.0f;
      sB0[kk][r] = (bval[i] && kin) ? Elem<T>::load(B0, bcol[i] + k0 + kk) : 0.0f;
      if constexpr (SWIGLU) sB1[kk][r] = (bval[i] && kin) ? Elem<T>::load(B1, bcol[i] + k0 + kk) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b0[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b0[j] = sB0[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
      if constexpr (SWIGLU) {
        float b1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[j] = sB1[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = ty * 4 + i;
    if (tr >= ti.rows) continue;
    const int64_t row = ti.row0 + tr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = nt * TN + tx * 4 + j;
      if (col >= p.Nout) continue;
      if constexpr (SWIGLU) {
        Elem<T>::store(static_cast<T*>(p.C), row * p.ldc + col, silu(acc0[i][j]) * acc1[i][j]);
      } else {
        static_cast<float*>(p.C)[split * p.c_split_stride + row * p.ldc + col] = acc0[i][j];
      }
    }
  }
}

template <typename T>
hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  const int64_t ntiles = (p.Nout + TN - 1) / TN;
  const int64_t mtiles = (p.rows_max + TM - 1) / TM + p.N;
  const int64_t blocks = ntiles * mtiles * p.splits;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (p.swiglu) {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_simple<T, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_simple<T, true, false>), grid, block, 0, s, p);
  } else {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_simple<T, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_simple<T, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_simple(const GemmParams& p, int bf16, hipStream_t s) {
  return bf16 ? launch_t<uint16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace moe
