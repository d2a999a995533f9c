// Gate-weighted combine back to token order, without atomics.
//
// y[t] = s * sum_{j=0..k-1, slot[t,j] >= 0} w[t,j] * y_perm[slot[t,j]]
// ("Llama 3 Meets MoE" review, section 3, MoE output; LLaMA-MoE v2 article,
// rescaling section). One workgroup per token gathers its k expert rows in
// slot order, so every output element is summed in the same fixed order; a
// dropped slot contributes nothing and a token with every slot dropped gets
// zeros. When the down projection was split over K, the partial rows are
// added in split order first.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Sum of one 4-column group over the token's kept slots, in slot order; the
// split-K partials of a row are added in split order first.
template <int KMAX>
__device__ __forceinline__ f32x4_t gather_sum(const CombineParams& p, const int (&sl)[KMAX], const float (&w)[KMAX],
                                              int64_t c) {
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4_t v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    v[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    if (sl[j] >= 0) {
      const float* src = p.y_perm + static_cast<int64_t>(sl[j]) * p.H + c * 4;
      v[j] = *reinterpret_cast<const f32x4_t*>(src);
      for (int s = 1; s < p.splits; ++s) v[j] += *reinterpret_cast<const f32x4_t*>(src + s * p.split_stride);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (sl[j] >= 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], v[j][q], acc[q]);
  return acc;
}

// y[t, 4c .. 4c+3] = s * acc
template <bool OUT_BF16>
__device__ __forceinline__ void store4(const CombineParams& p, int64_t t, int64_t c, f32x4_t acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] *= p.scale;
  if constexpr (OUT_BF16) {
    uint16_t* y = static_cast<uint16_t*>(p.y) + t * p.H + c * 4;
    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    *reinterpret_cast<uint2*>(y) = make_uint2(lo, hi);
  } else {
    *(reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + t * p.H) + c) = acc;
  }
}

template <bool OUT_BF16, int KMAX>
__global__ __launch_bounds__(256) void k_combine(CombineParams p) {
  const int64_t t = blockIdx.x;
  const int k = p.k, H = p.H;
  const int64_t H4 = H / 4;
  int sl[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    sl[j] = j < k ? p.slot[t * k + j] : -1;
    w[j] = j < k ? p.topk_w[t * k + j] : 0.0f;
  }
#pragma unroll 4
  for (int64_t c = threadIdx.x; c < H4; c += 256) store4<OUT_BF16>(p, t, c, gather_sum<KMAX>(p, sl, w, c));
}

// Any k: the same sums with the slots read inside the loop.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_combine_any(CombineParams p) {
  const int64_t t = blockIdx.x;
  const int k = p.k;
  const int64_t H4 = p.H / 4;
  for (int64_t c = threadIdx.x; c < H4; c += 256) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int sl = p.slot[t * k + j];
      if (sl < 0) continue;
      const float w = p.topk_w[t * k + j];
      const float* src = p.y_perm + static_cast<int64_t>(sl) * p.H + c * 4;
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
      for (int s = 1; s < p.splits; ++s) v += *reinterpret_cast<const f32x4_t*>(src + s * p.split_stride);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
    store4<OUT_BF16>(p, t, c, acc);
  }
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
