// Router on the matrix cores for bf16 activations.
//
// The router product x.W_g (and x.W_noise) is a skinny GEMM: T x H times
// H x N with N <= 64. The fp32 router weights are split exactly into three
// bf16 parts, W = W1 + W2 + W3 (each part holds the next 8 significant bits),
// so every product x * W_i of a bf16 activation is exact in fp32 and
// v_mfma_f32_16x16x32_bf16 forms x.W with fp32 accumulation. The hi part and
// the two lower parts go to separate accumulators and the four waves of a
// block each cover a quarter of H, which keeps the accumulated rounding error
// near that of a plain fp32 dot product.
//
// A block owns 16 tokens. After the product, one wave per token applies the
// noise term, KeepTopK by k rounds of a wave-wide argmax (ties to the lower
// expert index; "Llama 3 Meets MoE" review, section 3) and the gate of the
// chosen order (Mixtral: softmax over the kept scores; ST: softmax over all
// scores, section 5); threads of the block then sum the per-expert counts,
// gate weights and softmax(logit) values over the block's tokens in token
// order for the permutation and the balance statistics.
#include "common.h"
#include "kernels.h"

#include <algorithm>

typedef float f32x4_mma_t __attribute__((ext_vector_type(4)));

namespace moe {

namespace {

constexpr int kTok = 16;    // tokens per block (M of the MFMA)
// waves per block, each over 1/W of H: more waves for fewer output columns
// (shorter dependent load chains per wave), fewer when the partial sums of
// every wave would not fit in LDS
template <int NB16>
constexpr int router_waves() { return NB16 <= 2 ? 16 : (NB16 <= 4 ? 8 : 4); }

// Ws[p][c][h], p = 0..2, c < N2p (columns: W_g, then W_noise, then zero
// padding), K-contiguous bf16 bits.
__global__ __launch_bounds__(256) void k_router_wsplit(const float* __restrict__ Wg, const float* __restrict__ Wn,
                                                       int H, int N, int noisy, int N2p, uint16_t* __restrict__ Ws) {
  const int total = N2p * H;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int c = i / H, h = i - c * H;
    float w = 0.0f;
    if (c < N) w = Wg[static_cast<int64_t>(h) * N + c];
    else if (noisy && c < 2 * N) w = Wn[static_cast<int64_t>(h) * N + (c - N)];
    const uint16_t w1 = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(w1);
    const uint16_t w2 = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(w2);
    const uint16_t w3 = f32_to_bf16(r2);
    Ws[i] = w1;
    Ws[total + i] = w2;
    Ws[2 * total + i] = w3;
  }
}

template <int NB16>
__global__ __launch_bounds__(router_waves<NB16>() * 64) void k_router_mma(RouterParams p, int N2p) {
  constexpr int kWaves = router_waves<NB16>();
  constexpr int NC = NB16 * 16;
  __shared__ float s_part[kWaves][kTok][NC];
  __shared__ float s_log[kTok][NC];       // clean logits, then noise logits

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, H = p.H, k = p.k;
  const int64_t T = p.T;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
  const uint16_t* __restrict__ Ws = p.wsplit;
  const int64_t part = static_cast<int64_t>(N2p) * H;
  const int n2 = N * (p.noisy ? 2 : 1);  // real columns; the padding stays zero without loads

  // this wave's K range, in steps of 32
  const int steps = (H + 31) / 32;
  const int s0 = wave * steps / kWaves, s1 = (wave + 1) * steps / kWaves;
  const int row = lane & 15, kg = lane >> 4;  // A: token row; B: column; kg selects 8 of the 32 K
  const int64_t tok = tok0 + row;
  const bool tok_ok = tok < T;
  const uint16_t* xrow = x + (tok_ok ? tok : 0) * H;

  f32x4_mma_t acc_hi[NB16], acc_lo[NB16];
#pragma unroll
  for (int c = 0; c < NB16; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_hi[c][r] = acc_lo[c][r] = 0.0f;

  // The x loads of XU K steps go out together (one memory round trip for
  // the block's whole share of x at H = 4096); the weight parts, which stay
  // in L2, are loaded one step ahead of their MFMAs.
  constexpr int XU = NB16 == 2 ? 4 : 8;  // within 128 registers at 16 waves
  for (int s = s0; s < s1; s += XU) {
    bf16x8_t a[XU];
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int kk = (s + u) * 32 + kg * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if ((s + u) < s1 && kk < H && tok_ok) v = *reinterpret_cast<const u32x4_t*>(xrow + kk);
      a[u] = __builtin_bit_cast(bf16x8_t, v);
    }
    bf16x8_t b[2][NB16][3];
    auto load_w = [&](int u, int buf) {
      const int kk = (s + u) * 32 + kg * 8;
      const bool kin = (s + u) < s1 && kk < H;
#pragma unroll
      for (int c = 0; c < NB16; ++c)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          u32x4_t wv = {0u, 0u, 0u, 0u};
          if (kin && c * 16 + row < n2) wv = *reinterpret_cast<const u32x4_t*>(Ws + q * part + static_cast<int64_t>(c * 16 + row) * H + kk);
          b[buf][c][q] = __builtin_bit_cast(bf16x8_t, wv);
        }
    };
    load_w(0, 0);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      if (u + 1 < XU) load_w(u + 1, (u + 1) & 1);
#pragma unroll
      for (int c = 0; c < NB16; ++c) {
        acc_hi[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u & 1][c][0], acc_hi[c], 0, 0, 0);
        acc_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u & 1][c][1], acc_lo[c], 0, 0, 0);
        acc_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u & 1][c][2], acc_lo[c], 0, 0, 0);
      }
    }
  }
  // lane holds column (lane & 15) and token rows 4*(lane/16) + r
#pragma unroll
  for (int c = 0; c < NB16; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_part[wave][kg * 4 + r][c * 16 + row] = acc_hi[c][r] + acc_lo[c][r];
  __syncthreads();
  for (int i = threadIdx.x; i < kTok * NC; i += kWaves * 64) {
    const int t = i / NC, c = i % NC;
    float v = s_part[0][t][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_part[w][t][c];
    s_log[t][c] = v;
  }
  __syncthreads();

  // one wave per token, lane n holding expert n: noise, KeepTopK, gates
  __shared__ float s_sel[kTok][64];  // gate weight of expert n if kept, else 0
  __shared__ int s_take[kTok][64];   // 1 if expert n is among the token's top k
  __shared__ float s_p[kTok][64];    // softmax of the clean logits
  const bool valid = lane < N;
  for (int t = wave; t < kTok; t += kWaves) {
    const int64_t g = tok0 + t;
    if (g >= T) break;  // wave-uniform
    const float lv = valid ? s_log[t][lane] : -INFINITY;
    float hv = lv;
    // H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i), the
    // normal draw being the input eps[t, i]
    if (p.noisy && valid) hv = fmaf(p.eps[g * N + lane], softplus(s_log[t][N + lane]), lv);
    if (p.logits && valid) p.logits[g * N + lane] = lv;
    // KeepTopK: k rounds of a wave-wide (score desc, index asc) argmax
    float cur = valid ? hv : -INFINITY;
    int curi = valid ? lane : 4096 + lane;
    bool taken = false;
    float my_v = 0.0f;
    int my_i = 0;
    for (int jj = 0; jj < k; ++jj) {
      float bv = cur;
      int bi = curi;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == jj) {
        my_v = bv;
        my_i = bi;
      }
      if (curi == bi) {
        taken = true;
        cur = -INFINITY;
        curi = 8192 + lane;
      }
    }
    const float hmax = __shfl(my_v, 0, 64);
    // Mixtral order: softmax over the kept scores; ST: over all N scores
    const float den = p.order == 0 ? wave_sum(lane < k ? expf(my_v - hmax) : 0.0f)
                                   : wave_sum(valid ? expf(hv - hmax) : 0.0f);
    if (lane < k) {
      p.topk_idx[g * k + lane] = my_i;
      p.topk_w[g * k + lane] = expf(my_v - hmax) / den;
    }
    s_take[t][lane] = taken ? 1 : 0;
    s_sel[t][lane] = taken ? expf(hv - hmax) / den : 0.0f;  // the value written for this expert
    if (p.stat_part) {
      const float lmax = wave_max(lv);
      const float el = valid ? expf(lv - lmax) : 0.0f;
      s_p[t][lane] = el / wave_sum(el);
    }
  }
  __syncthreads();

  // per-block sums over the tokens, in token order
  if (p.hist && threadIdx.x < N) {
    const int n = threadIdx.x;
    int cnt = 0;
    float imp = 0.0f, ps = 0.0f;
    for (int t = 0; t < kTok; ++t) {
      if (tok0 + t >= T) break;
      cnt += s_take[t][n];
      imp += s_sel[t][n];
      if (p.stat_part) ps += s_p[t][n];
    }
    p.hist[static_cast<int64_t>(blockIdx.x) * N + n] = cnt;
    if (p.stat_part) {
      p.stat_part[static_cast<int64_t>(blockIdx.x) * 2 * N + 2 * n] = imp;
      p.stat_part[static_cast<int64_t>(blockIdx.x) * 2 * N + 2 * n + 1] = ps;
    }
  }
}

}  // namespace

int router_mma_columns(int N, int noisy) {
  const int n2 = N * (noisy ? 2 : 1);
  return (n2 + 15) / 16 * 16;
}

size_t router_wsplit_bytes(int H, int N, int noisy) {
  return static_cast<size_t>(3) * router_mma_columns(N, noisy) * H * sizeof(uint16_t);
}

hipError_t launch_router_mma(const RouterParams& p, hipStream_t s) {
  const int N2p = router_mma_columns(p.N, p.noisy);
  {
    const int64_t total = static_cast<int64_t>(N2p) * p.H;
    const int blocks = static_cast<int>(std::min<int64_t>((total + 255) / 256, 2048));
    hipLaunchKernelGGL(k_router_wsplit, dim3(blocks), dim3(256), 0, s, p.Wg, p.Wn, p.H, p.N, p.noisy, N2p, p.wsplit);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>((p.T + kTok - 1) / kTok));
#define MOE_ROUTER_MMA(NB) \
  hipLaunchKernelGGL(k_router_mma<NB>, grid, dim3(router_waves<NB>() * 64), 0, s, p, N2p)
  switch (N2p / 16) {
    case 1: MOE_ROUTER_MMA(1); break;
    case 2: MOE_ROUTER_MMA(2); break;
    case 3: MOE_ROUTER_MMA(3); break;
    case 4: MOE_ROUTER_MMA(4); break;
    case 5: MOE_ROUTER_MMA(5); break;
    case 6: MOE_ROUTER_MMA(6); break;
    case 7: MOE_ROUTER_MMA(7); break;
    default: MOE_ROUTER_MMA(8); break;
  }
#undef MOE_ROUTER_MMA
  return hipGetLastError();
}

}  // namespace moe
