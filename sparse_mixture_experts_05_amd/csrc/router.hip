// Router, KeepTopK and gate weights for the MoE layer on gfx950.
//
// One wavefront owns TPW tokens. Lanes stride the hidden dimension in
// 16-byte pieces (8 elements), accumulate x.W_g (and x.W_noise) for all
// experts in fp32 registers, and a butterfly over the 64 lanes finishes the
// dot products. Lane n then holds the score of expert n; k rounds of a
// wave-wide (score desc, index asc) argmax give KeepTopK with ties to the
// lower index ("Llama 3 Meets MoE" review, section 3, KeepTopK), and the gate
// weights follow either the Mixtral order (softmax over the kept scores) or
// the ST order (softmax over all scores, read at the kept experts; review,
// section 5). Per-block expert counts, gate-weight sums and softmax(logit)
// sums are written for the permutation and the balance statistics.
#include "common.h"
#include "kernels.h"
#include "stats.h"

namespace moe {

namespace {

constexpr int kRouterWaves = 4;

template <int NMAX>
constexpr int router_tpw() { return NMAX <= 16 ? 4 : (NMAX == 32 ? 2 : 1); }

template <typename XT>
__device__ __forceinline__ void load8(const XT* row, int h, float* out);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* row, int h, float* out) {
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + h);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* row, int h, float* out) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(row + h);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(row + h + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

// acc[t][n] += sum_i xv[t][i] * W[(h+i)*N + n]
template <int NMAX, int TPW, bool VEC4>
__device__ __forceinline__ void accumulate(const float* __restrict__ W, int h, int N, const float (&xv)[TPW][8],
                                           float (&acc)[TPW][NMAX]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float* wrow = W + static_cast<int64_t>(h + i) * N;
    if constexpr (VEC4) {
#pragma unroll
      for (int n = 0; n < NMAX; n += 4) {
        if (n < N) {
          const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wrow + n);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t][n + q] = fmaf(xv[t][i], w4[q], acc[t][n + q]);
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        if (n < N) {
          const float w = wrow[n];
#pragma unroll
          for (int t = 0; t < TPW; ++t) acc[t][n] = fmaf(xv[t][i], w, acc[t][n]);
        }
      }
    }
  }
}

template <int NMAX, bool NOISY, typename XT, bool VEC4>
__global__ __launch_bounds__(kRouterWaves * kWave) void k_router(RouterParams p) {
  constexpr int TPW = router_tpw<NMAX>();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int N = p.N, H = p.H, k = p.k;
  const int64_t T = p.T;
  const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * kRouterWaves + wave) * TPW;
  const XT* __restrict__ x = static_cast<const XT*>(p.x);

  float acc[TPW][NMAX];
  float nacc[NOISY ? TPW : 1][NOISY ? NMAX : 1];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int n = 0; n < NMAX; ++n) acc[t][n] = 0.0f;
  if constexpr (NOISY) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int n = 0; n < NMAX; ++n) nacc[t][n] = 0.0f;
  }

  // x . W_g (and x . W_noise), each lane over its slice of H
  for (int h = lane * 8; h < H; h += 8 * kWave) {
    float xv[TPW][8];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (tok0 + t < T) {
        load8<XT>(x + (tok0 + t) * H, h, xv[t]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[t][i] = 0.0f;
      }
    }
    accumulate<NMAX, TPW, VEC4>(p.Wg, h, N, xv, acc);
    if constexpr (NOISY) accumulate<NMAX, TPW, VEC4>(p.Wn, h, N, xv, nacc);
  }

  float cnt = 0.0f, imp = 0.0f, psum = 0.0f, slsum = 0.0f;  // this lane's expert, summed over the wave's tokens
  const bool valid = lane < N;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t tok = tok0 + t;
    if (tok >= T) break;  // wave-uniform
    float lv = -INFINITY, nz = 0.0f;
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      if (n < N) {
        const float s = wave_sum(acc[t][n]);
        if (lane == n) lv = s;
        if constexpr (NOISY) {
          const float z = wave_sum(nacc[t][n]);
          if (lane == n) nz = z;
        }
      }
    }
    float hv = lv;
    if constexpr (NOISY) {
      // H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i); the
      // normal draw is the input eps[t, i]
      if (valid) hv = fmaf(p.eps[tok * N + lane], softplus(nz), lv);
    }
    // a NaN score counts as -inf in KeepTopK and the gates: the argmax below
    // then compares a strict total order, so every lane agrees on the winner
    if (hv != hv) hv = -INFINITY;
    if (p.logits && valid) p.logits[tok * N + lane] = lv;
    if constexpr (NOISY) {
      if (p.noise_logits && valid) p.noise_logits[tok * N + lane] = nz;
    }

    // KeepTopK: k rounds of a wave-wide argmax, ties to the lower index
    float cur = valid ? hv : -INFINITY;
    int curi = valid ? lane : 4096;
    bool taken = false;
    float my_v = 0.0f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
      float bv = cur;
      int bi = curi;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == j) {
        my_v = bv;
        my_i = bi;
      }
      if (curi == bi) {
        taken = true;
        cur = -INFINITY;
        curi = 4096 + lane;
      }
    }
    // smooth load (Shazeer et al. 2017, the TopK Noisy Gate the LLaMA-MoE hub
    // page names): Phi((clean logit - k-th highest other score) /
    // Softplus(noise logit)); that score is the k-th highest overall for an
    // expert not kept, the (k+1)-th (one more argmax round; -inf when k = N)
    // for a kept one
    float sl = 0.0f;
    if constexpr (NOISY) {
      if (p.smooth && p.stat_part) {
        const float vk = __shfl(my_v, k - 1, kWave);
        float vk1 = -INFINITY;
        if (k < N) {
          float bv = cur;
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) bv = fmaxf(bv, __shfl_xor(bv, m, kWave));
          vk1 = bv;
        }
        const float z = (lv - (taken ? vk1 : vk)) / softplus(nz);
        sl = valid ? 0.5f * erfcf(z * -0.70710678118654752f) : 0.0f;
      }
    }
    const float hmax = __shfl(my_v, 0, kWave);
    float den;
    if (p.order == 0) {
      // Mixtral order: softmax over the kept scores
      den = wave_sum(lane < k ? expf(my_v - hmax) : 0.0f);
    } else {
      // ST order: softmax over all N scores, not renormalised after top-k
      den = wave_sum(valid ? expf(hv - hmax) : 0.0f);
    }
    if (lane < k) {
      p.topk_idx[tok * k + lane] = my_i;
      p.topk_w[tok * k + lane] = expf(my_v - hmax) / den;
    }
    if (p.hist) {
      cnt += taken ? 1.0f : 0.0f;
      if (taken) imp += expf(hv - hmax) / den;  // same value as written for this expert
      if (p.stat_part) {
        // mean of softmax(clean logits) for P
        const float lmax = wave_max(lv);
        const float el = valid ? expf(lv - lmax) : 0.0f;
        const float dl = wave_sum(el);
        psum += el / dl;
        slsum += sl;
      }
    }
  }

  if (p.hist) {
    __shared__ float red[kRouterWaves][4][64];
    red[wave][0][lane] = cnt;
    red[wave][1][lane] = imp;
    red[wave][2][lane] = psum;
    red[wave][3][lane] = slsum;
    __syncthreads();
    if (threadIdx.x < N) {
      const int n = threadIdx.x;
      float c = 0.0f, s_imp = 0.0f, s_p = 0.0f, s_sl = 0.0f;
#pragma unroll
      for (int w = 0; w < kRouterWaves; ++w) {
        c += red[w][0][n];
        s_imp += red[w][1][n];
        s_p += red[w][2][n];
        s_sl += red[w][3][n];
      }
      p.hist[static_cast<int64_t>(blockIdx.x) * N + n] = static_cast<int32_t>(c);
      if (p.stat_part) {
        float* part = p.stat_part + (static_cast<int64_t>(blockIdx.x) * N + n) * kStatsPerExpert;
        part[0] = s_imp;
        part[1] = s_p;
        part[2] = s_sl;
      }
    }
  }
}

template <int NMAX>
hipError_t launch_router_n(const RouterParams& p, hipStream_t s) {
  const dim3 grid(router_blocks(p.T, p.N, p.noisy, 0)), block(kRouterWaves * kWave);
  const bool vec4 = (p.N % 4) == 0;
#define MOE_ROUTER_LAUNCH(NOISY, XT, V4) \
  hipLaunchKernelGGL((k_router<NMAX, NOISY, XT, V4>), grid, block, 0, s, p)
  if (p.noisy) {
    if (p.act_bf16) {
      if (vec4) MOE_ROUTER_LAUNCH(true, uint16_t, true); else MOE_ROUTER_LAUNCH(true, uint16_t, false);
    } else {
      if (vec4) MOE_ROUTER_LAUNCH(true, float, true); else MOE_ROUTER_LAUNCH(true, float, false);
    }
  } else {
    if (p.act_bf16) {
      if (vec4) MOE_ROUTER_LAUNCH(false, uint16_t, true); else MOE_ROUTER_LAUNCH(false, uint16_t, false);
    } else {
      if (vec4) MOE_ROUTER_LAUNCH(false, float, true); else MOE_ROUTER_LAUNCH(false, float, false);
    }
  }
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

int nmax_for(int N) { return N <= 8 ? 8 : N <= 16 ? 16 : N <= 32 ? 32 : 64; }

// The fixed-order statistics reduction (stats.h) in a workgroup of its own.
__global__ __launch_bounds__(kStatGroups * 64) void k_stats(StatsParams p) {
  __shared__ __attribute__((aligned(16))) char s_lds[kStatLdsBytes];
  stats_reduce(p, s_lds);
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}
__global__ void k_fill_f32(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

int router_tokens_per_block(int N, int /*noisy*/, int act_bf16) {
  if (act_bf16) return 16;  // the matrix-core router (router_mma.hip)
  const int nm = nmax_for(N);
  const int tpw = nm <= 16 ? 4 : (nm == 32 ? 2 : 1);
  return tpw * kRouterWaves;
}

int router_blocks(int64_t T, int N, int noisy, int act_bf16) {
  const int tpb = router_tokens_per_block(N, noisy, act_bf16);
  return static_cast<int>((T + tpb - 1) / tpb);
}

hipError_t launch_router(const RouterParams& p, hipStream_t s) {
  if (p.act_bf16) return launch_router_mma(p, s);
  switch (nmax_for(p.N)) {
    case 8: return launch_router_n<8>(p, s);
    case 16: return launch_router_n<16>(p, s);
    case 32: return launch_router_n<32>(p, s);
    default: return launch_router_n<64>(p, s);
  }
}

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_stats, dim3(1), dim3(kStatGroups * 64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* ptr, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = static_cast<int>(n < 256 * 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks), dim3(256), 0, s, ptr, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* ptr, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = static_cast<int>(n < 256 * 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(k_fill_f32, dim3(blocks), dim3(256), 0, s, ptr, n, v);
  return hipGetLastError();
}

}  // namespace moe
