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

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_combine(CombineParams p) {
  const int64_t t = blockIdx.x;
  const int k = p.k, H = p.H;
  const int64_t H4 = H / 4;
  for (int64_t c = threadIdx.x; c < H4; c += 256) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int sl = p.slot[t * k + j];
      if (sl < 0) continue;
      const float w = p.topk_w[t * k + j];
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.y_perm + static_cast<int64_t>(sl) * H) + c;
      f32x4_t v = src[0];
      for (int s = 1; s < p.splits; ++s) v += *reinterpret_cast<const f32x4_t*>(
                                                  reinterpret_cast<const float*>(src) + s * p.split_stride);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] *= p.scale;
    if constexpr (OUT_BF16) {
      uint16_t* y = static_cast<uint16_t*>(p.y) + t * H + c * 4;
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
      *reinterpret_cast<uint2*>(y) = make_uint2(lo, hi);
    } else {
      *(reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + t * H) + c) = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.T)), block(256);
  if (p.out_bf16) hipLaunchKernelGGL(k_combine<true>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(k_combine<false>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
