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

// Non-temporal cache policy of the buffer accesses (every y_perm element is
// read once and every y element written once).
constexpr int kNT = 2;

template <bool OUT_BF16, int KMAX>
__global__ __launch_bounds__(256) void k_combine(CombineParams p) {
  const int64_t t = blockIdx.x;
  const int k = p.k, H = p.H;
  const int64_t H4 = H / 4;
  // the token's slots and weights, requested together with the error word
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(p.slot + t * k, static_cast<int64_t>(k) * 4);
  const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(p.topk_w + t * k, static_cast<int64_t>(k) * 4);
  int sl[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    sl[j] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rs, j * 4u, 0, 0));
    w[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, j * 4u, 0, 0));
  }
  if (poisoned<OUT_BF16>(p, t)) return;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) sl[j] = j < k ? checked_slot(sl[j], p.rows, p.dbg, kDbgCombineSlot) : -1;
  if (p.splits > 1 || p.res_splits > 1) {
    // split-K partial rows (decode shapes): added in split order first
#pragma unroll 4
    for (int64_t c = threadIdx.x; c < H4; c += 256) cmb::store4<OUT_BF16>(p, t, c, cmb::gather_sum<KMAX>(p, sl, w, c));
    return;
  }
  // up to four 4-column groups per thread: every kept row's groups (and the
  // residual's) are requested before any y store, since a load issued after
  // a store would also wait for that store; a dropped slot's offsets are out
  // of range and read zeros
  constexpr int kP = KMAX <= 4 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t ry = uniform_rsrc(p.y_perm, p.rows * H * 4);
  const __amdgpu_buffer_rsrc_t rr = uniform_rsrc(p.residual ? p.residual + t * H : p.y_perm, p.residual ? H * 4 : 0);
  for (int64_t c0 = threadIdx.x; c0 < H4; c0 += kP * 256) {
    f32x4_t v[kP][KMAX], r[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int64_t c = c0 + i * 256;
      const bool cv = c < H4;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const uint32_t off = (cv && sl[j] >= 0) ? static_cast<uint32_t>(sl[j] * H + c * 4) * 4u : kOOB;
        v[i][j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, kNT));
      }
      r[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rr, cv ? static_cast<uint32_t>(c) * 16u : kOOB, 0, kNT));
    }
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int64_t c = c0 + i * 256;
      if (c >= H4) break;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (sl[j] >= 0)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], v[i][j][q], acc[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = p.residual ? fmaf(p.scale, acc[q], r[i][q]) : acc[q] * p.scale;
      if constexpr (OUT_BF16) {
        const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[0])) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[2])) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        uint16_t* y = static_cast<uint16_t*>(p.y) + t * H + c * 4;
        __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(y));
      } else {
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + t * H) + c);
      }
    }
  }
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
