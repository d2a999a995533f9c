// Gate-weighted combine of one token's kept expert rows: the forms the
// combine kernel uses for split-K partial rows and for more than eight slots.
//
// y[t] = s * sum_{j=0..k-1, slot[t,j] >= 0} w[t,j] * y_perm[slot[t,j]]
// ("Llama 3 Meets MoE" review, section 3, MoE output; LLaMA-MoE v2 article,
// rescaling section), summed in slot order, so every element is the same on
// every run; a dropped slot contributes nothing and a token with every slot
// dropped gets zeros. When the down projection was split over K, the partial
// rows are added in split order first.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {
namespace cmb {

// Every y_perm element is read once and every y element written once, so
// both go through non-temporal accesses (same values; at the 2/8 and 4/16
// LLaMA-MoE shapes the layer runs 1.4% and 2.4% faster than with the default
// cache policy).
__device__ __forceinline__ f32x4_t ld_nt(const float* src) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src));
}

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
      v[j] = ld_nt(src);
      for (int s = 1; s < p.splits; ++s) v[j] += ld_nt(src + s * p.split_stride);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (sl[j] >= 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], v[j][q], acc[q]);
  return acc;
}

// y[t, 4c .. 4c+3] = s * acc, or residual + s * acc for the residual layer
// (its shared slice's partial rows added in split order first)
template <bool OUT_BF16>
__device__ __forceinline__ void store4(const CombineParams& p, int64_t t, int64_t c, f32x4_t acc) {
  if (p.residual) {
    const float* src = p.residual + t * p.H + c * 4;
    f32x4_t r = ld_nt(src);
    for (int s = 1; s < p.res_splits; ++s) r += ld_nt(src + s * p.res_split_stride);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(p.scale, acc[q], r[q]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] *= p.scale;
  }
  if constexpr (OUT_BF16) {
    uint16_t* y = static_cast<uint16_t*>(p.y) + t * p.H + c * 4;
    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(y));
  } else {
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + t * p.H) + c);
  }
}

// Any k: the same sums with the slots read inside the loop; lanes `lane`,
// `lane + nl`, ... of a group of nl lanes each take every nl-th 4-column group.
template <bool OUT_BF16>
__device__ __forceinline__ void token_any(const CombineParams& p, int64_t t, int lane, int nl) {
  const int k = p.k;
  const int64_t H4 = p.H / 4;
  for (int64_t c = lane; c < H4; c += nl) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const int sl = checked_slot(p.slot[t * k + j], p.rows, p.dbg, kDbgCombineSlot);
      if (sl < 0) continue;
      const float w = p.topk_w[t * k + j];
      const float* src = p.y_perm + static_cast<int64_t>(sl) * p.H + c * 4;
      f32x4_t v = ld_nt(src);
      for (int s = 1; s < p.splits; ++s) v += ld_nt(src + s * p.split_stride);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
    store4<OUT_BF16>(p, t, c, acc);
  }
}

}  // namespace cmb
}  // namespace moe
