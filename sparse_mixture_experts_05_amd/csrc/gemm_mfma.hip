// Grouped bf16 GEMMs of the SwiGLU experts on gfx950 matrix cores.
//
// Rows of expert e occupy [offsets[e], offsets[e+1]) of the permuted order.
// A workgroup owns one BM x BN output tile of one expert; it finds its expert
// on the device from `offsets` (no host synchronisation), stages A and B
// tiles of BK = 64 through LDS with double buffering, and issues
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
//   swiglu: B rows [0, BN/2) are Wgate rows, [BN/2, BN) the matching Wup rows;
//           each wave holds gate and up accumulators of the same columns, so
//           the epilogue forms SiLU(g) * u in registers and stores h as bf16
//           (LLaMA-MoE v2 article, code example, class Expert).
//   plain : C = A . B^T in fp32 (the down projection), optionally split over K
//           into separate partial outputs that the combine step adds in a
//           fixed order.
//
// Both operands are K-contiguous ("TN"): a 16-byte LDS read gives a lane its
// 8 bf16 MFMA operand elements. LDS rows are 128 bytes (BK bf16); the 16-byte
// chunk c of row r is stored at chunk c ^ (r & 7), which keeps both the
// row-wise global->LDS writes and the column-wise MFMA operand reads free of
// bank conflicts.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <int BM, int BN, int WGM, int WGN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm_mfma(GemmParams p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int CA = BM * 8 / NT, CB = BN * 8 / NT;  // 16-byte chunks per thread per K step
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!SWIGLU || NB % 2 == 0, "swiglu needs gate/up block pairs");
  static_assert(CA >= 1 && CB >= 1 && (BM * 8) % NT == 0 && (BN * 8) % NT == 0, "load split");

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int NO = SWIGLU ? BN / 2 : BN;  // output columns per tile
  const int ntiles = (p.Nout + NO - 1) / NO;
  const int mtiles = static_cast<int>((p.rows_max + BM - 1) / BM) + p.N;
  int bid = blockIdx.x;
  const int nt = bid % ntiles;
  bid /= ntiles;
  const int mt = bid % mtiles;
  const int split = bid / mtiles;

  TileInfo ti;
  if (!find_tile<BM>(p.offsets, p.N, mt, ti)) return;  // uniform over the workgroup

  // K range of this split
  const int kper = ((p.K + p.splits - 1) / p.splits + BK - 1) / BK * BK;
  const int kb0 = split * kper;
  const int kb1 = min(p.K, kb0 + kper);
  const int KT = kb1 > kb0 ? (kb1 - kb0 + BK - 1) / BK : 0;

  // per-thread global source rows
  const uint16_t* __restrict__ Ab = static_cast<const uint16_t*>(p.A);
  const uint16_t* arow[CA];
  int achunk[CA];
  bool aval[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int ci = tid + i * NT;
    const int r = ci >> 3;
    achunk[i] = ci & 7;
    aval[i] = r < ti.rows;
    int64_t src = ti.row0 + r;
    if (GATHER) src = aval[i] ? p.row_token[src] : 0;
    arow[i] = Ab + (aval[i] ? src : 0) * p.lda;
  }
  const uint16_t* __restrict__ B0 = static_cast<const uint16_t*>(p.B0) + ti.expert * p.b_expert_stride;
  const uint16_t* __restrict__ B1 = SWIGLU ? static_cast<const uint16_t*>(p.B1) + ti.expert * p.b_expert_stride : nullptr;
  const uint16_t* brow[CB];
  int bchunk[CB];
  bool bval[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int ci = tid + i * NT;
    const int r = ci >> 3;
    bchunk[i] = ci & 7;
    int f;
    const uint16_t* base;
    if (SWIGLU) {
      const bool up = r >= BN / 2;
      f = nt * NO + (up ? r - BN / 2 : r);
      base = up ? B1 : B0;
    } else {
      f = nt * NO + r;
      base = B0;
    }
    bval[i] = f < p.Nout;
    brow[i] = base + static_cast<int64_t>(bval[i] ? f : 0) * p.ldb;
  }

  u32x4_t ra[CA], rb[CB];
  auto gload = [&](int kt) {
    const int kb = kb0 + kt * BK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int kk = kb + achunk[i] * 8;
      if (aval[i] && kk < kb1) ra[i] = *reinterpret_cast<const u32x4_t*>(arow[i] + kk);
      else ra[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int kk = kb + bchunk[i] * 8;
      if (bval[i] && kk < kb1) rb[i] = *reinterpret_cast<const u32x4_t*>(brow[i] + kk);
      else rb[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int r = (tid + i * NT) >> 3;
      *reinterpret_cast<u32x4_t*>(&sA[buf][swz(r, achunk[i])]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int r = (tid + i * NT) >> 3;
      *reinterpret_cast<u32x4_t*>(&sB[buf][swz(r, bchunk[i])]) = rb[i];
    }
  };

  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // B rows read by this wave's blocks
  int brow_l[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (SWIGLU) {
      const int half = NB / 2;
      const int jj = j < half ? j : j - half;
      brow_l[j] = (j < half ? 0 : BN / 2) + wn * (WN / 2) + jj * 32 + (lane & 31);
    } else {
      brow_l[j] = wn * WN + j * 32 + (lane & 31);
    }
  }
  int arow_l[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) arow_l[i] = wm * WM + i * 32 + (lane & 31);
  const int khalf = lane >> 5;

  if (KT > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + khalf;
      bf16x8_t af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][swz(arow_l[i], chunk)]);
#pragma unroll
      for (int j = 0; j < NB; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[cur][swz(brow_l[j], chunk)]);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
  const int col_l = lane & 31;
  if (SWIGLU) {
    uint16_t* __restrict__ C = static_cast<uint16_t*>(p.C);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        const int f = nt * NO + wn * (WN / 2) + j * 32 + col_l;
        if (f >= p.Nout) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = wm * WM + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
          if (tr < ti.rows) {
            const float g = acc[i][j][r], u = acc[i][j + NB / 2][r];
            C[static_cast<int64_t>(ti.row0 + tr) * p.ldc + f] = f32_to_bf16(silu(g) * u);
          }
        }
      }
  } else {
    float* __restrict__ C = static_cast<float*>(p.C) + split * p.c_split_stride;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = nt * NO + wn * WN + j * 32 + col_l;
        if (n >= p.Nout) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tr = wm * WM + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
          if (tr < ti.rows) C[static_cast<int64_t>(ti.row0 + tr) * p.ldc + n] = acc[i][j][r];
        }
      }
  }
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  const int NO = p.swiglu ? BN / 2 : BN;
  const int64_t ntiles = (p.Nout + NO - 1) / NO;
  const int64_t mtiles = (p.rows_max + BM - 1) / BM + p.N;
  const int64_t blocks = ntiles * mtiles * p.splits;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), block(WGM * WGN * 64);
  if (p.swiglu) {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, true, false>), grid, block, 0, s, p);
  } else {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_mfma_supported(int K, int Nout) { return K % 8 == 0 && K > 0 && Nout > 0; }

hipError_t launch_gemm_bf16_mfma(const GemmParams& p, hipStream_t s) {
  // few rows per expert: short, wide tiles; otherwise square tiles
  const int64_t avg_rows = p.rows_max / (p.N > 0 ? p.N : 1);
  if (avg_rows <= 48) return launch_cfg<32, 256, 1, 4>(p, s);
  return launch_cfg<128, 128, 2, 2>(p, s);
}

}  // namespace moe
