// Gate-weighted combine back to token order, without atomics: one workgroup
// per token gathers its k expert rows in slot order (combine.h).
#include "combine.h"

namespace moe {

namespace {

// When an earlier kernel of the layer reported a failure (a bounded wait that
// gave up), the whole output is NaN, so the failure cannot pass as a result.
template <bool OUT_BF16>
__device__ __forceinline__ bool poisoned(const CombineParams& p, int64_t t) {
  if (!p.error || *p.error == 0) return false;
  const f32x4_t nan4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  for (int64_t c = threadIdx.x; c < p.H / 4; c += blockDim.x) {
    const f32x4_t v = nan4;
    cmb::store4<OUT_BF16>(p, t, c, v);
  }
  return true;
}

template <bool OUT_BF16, int KMAX>
__global__ __launch_bounds__(256) void k_combine(CombineParams p) {
  const int64_t t = blockIdx.x;
  const int k = p.k, H = p.H;
  const int64_t H4 = H / 4;
  if (poisoned<OUT_BF16>(p, t)) return;
  int sl[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    sl[j] = j < k ? checked_slot(p.slot[t * k + j], p.rows, p.dbg, kDbgCombineSlot) : -1;
    w[j] = j < k ? p.topk_w[t * k + j] : 0.0f;
  }
#pragma unroll 4
  for (int64_t c = threadIdx.x; c < H4; c += 256) cmb::store4<OUT_BF16>(p, t, c, cmb::gather_sum<KMAX>(p, sl, w, c));
}

// Any k: the same sums with the slots read inside the loop.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_combine_any(CombineParams p) {
  if (poisoned<OUT_BF16>(p, blockIdx.x)) return;
  cmb::token_any<OUT_BF16>(p, blockIdx.x, threadIdx.x, 256);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.T)), block(256);
#define MOE_COMBINE(KMAX)                                                          \
  do {                                                                             \
    if (p.out_bf16) hipLaunchKernelGGL((k_combine<true, KMAX>), grid, block, 0, s, p); \
    else hipLaunchKernelGGL((k_combine<false, KMAX>), grid, block, 0, s, p);       \
  } while (0)
  if (p.k <= 2) MOE_COMBINE(2);
  else if (p.k <= 4) MOE_COMBINE(4);
  else if (p.k <= 8) MOE_COMBINE(8);
  else if (p.out_bf16) hipLaunchKernelGGL(k_combine_any<true>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(k_combine_any<false>, grid, block, 0, s, p);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
