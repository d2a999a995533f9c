// Router on the matrix cores for bf16 activations.
//
// The router product x.W_g (and x.W_noise) is a skinny GEMM: T x H times
// H x N with N <= 64. Each fp32 router weight is split exactly into three
// bf16 parts, W = W1 + W2 + W3 (each part holds the next 8 significant bits;
// round-to-nearest-even leaves a remainder that the next part holds exactly),
// so every product x * W_i of a bf16 activation is exact in fp32 and
// v_mfma_f32_16x16x32_bf16 forms x.W with fp32 accumulation. The hi part and
// the two lower parts go to separate accumulators and the waves of a block
// each cover a share of H, which keeps the accumulated rounding error near
// that of a plain fp32 dot product.
//
// A block owns 16 tokens. It walks H in chunks: the chunk's fp32 weight rows
// are copied into LDS with coalesced loads (issued together with the x loads),
// and each lane reads its eight operand values per K step from LDS and splits
// them in registers. After the product, one wave per token applies the
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

constexpr int kWFloats = 32 * 1024;  // LDS for one chunk of fp32 weight rows (128 KB)
// most K steps of one wave in one chunk (their x loads stay in registers)
template <int NB16>
constexpr int router_xu() { return NB16 == 2 ? 4 : 8; }

// Rows of H per chunk: a multiple of 32 * waves (whole K steps for every
// wave), at most kXU steps per wave, and within kWFloats for all n2 columns.
constexpr int kWPad = 4;             // floats of padding per LDS column

template <int NB16>
int router_chunk_rows(int H, int n2) {
  const int unit = 32 * router_waves<NB16>();
  int rows = kWFloats / n2 / unit * unit;
  rows = std::min(rows, router_xu<NB16>() * unit);
  rows = std::max(rows, unit);
  return std::min(rows, (H + unit - 1) / unit * unit);
}

// Exact three-way bf16 split of eight fp32 values.
__device__ __forceinline__ void split3(const float (&w)[8], bf16x8_t& p1, bf16x8_t& p2, bf16x8_t& p3) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 b1 = static_cast<__bf16>(w[i]);
    const float r1 = w[i] - static_cast<float>(b1);
    const __bf16 b2 = static_cast<__bf16>(r1);
    const float r2 = r1 - static_cast<float>(b2);
    p1[i] = b1;
    p2[i] = b2;
    p3[i] = static_cast<__bf16>(r2);
  }
}

template <int NB16>
__global__ __launch_bounds__(router_waves<NB16>() * 64) void k_router_mma(RouterParams p, int hc) {
  constexpr int kWaves = router_waves<NB16>();
  constexpr int kThreads = kWaves * 64;
  constexpr int NC = NB16 * 16;
  constexpr int kXU = router_xu<NB16>();
  // the weight chunk; after the product, the per-wave partial sums
  // (n2 <= 128 padded columns of at most kWFloats / n2 rows)
  __shared__ __attribute__((aligned(16))) float s_w[kWFloats + kWPad * 128];
  static_assert(kWaves * kTok * NC <= kWFloats, "partials fit in the weight buffer");
  float (*s_part)[kTok][NC] = reinterpret_cast<float (*)[kTok][NC]>(s_w);
  __shared__ float s_log[kTok][NC];       // clean logits, then noise logits

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, H = p.H, k = p.k;
  const int64_t T = p.T;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
  const int n2 = N * (p.noisy ? 2 : 1);  // real columns; the padding stays zero

  const int row = lane & 15, kg = lane >> 4;  // A: token row; B: column; kg selects 8 of the 32 K
  const int64_t tok = tok0 + row;
  const bool tok_ok = tok < T;
  const uint16_t* xrow = x + (tok_ok ? tok : 0) * H;
  const int wsteps = hc / 32 / kWaves;  // this wave's K steps per chunk

  f32x4_mma_t acc_hi[NB16], acc_lo[NB16];
#pragma unroll
  for (int c = 0; c < NB16; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_hi[c][r] = acc_lo[c][r] = 0.0f;

  // 16-byte weight loads need aligned pointers and whole rows per piece
  const bool vec = (reinterpret_cast<uintptr_t>(p.Wg) & 15) == 0 &&
                   (!p.noisy || (reinterpret_cast<uintptr_t>(p.Wn) & 15) == 0) && N % 4 == 0;
  const int hcp = hc + kWPad;  // LDS column stride: column j of the chunk holds its rows k contiguous
  for (int h0 = 0; h0 < H; h0 += hc) {
    const int hn = min(hc, H - h0);  // weight rows in this chunk
    // the chunk's weight rows go to LDS transposed, W_g as columns [0, N) and
    // W_noise as columns [N, 2N): 16-byte pieces, all of a thread's loads out
    // before any store
    const int cnt = hn * N, c4 = vec ? cnt / 4 : 0, np = (p.noisy ? 2 : 1) * c4;
    constexpr int kP = kWFloats / 4 / kThreads;  // most pieces per thread
    f32x4_t wbuf[kP];
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < np) {
        const int m = i < c4 ? 0 : 1, q = i - m * c4;
        wbuf[j] = *reinterpret_cast<const f32x4_t*>((m == 0 ? p.Wg : p.Wn) + static_cast<int64_t>(h0) * N + 4 * q);
      }
    }
    // x of this wave's steps in the chunk
    bf16x8_t a[kXU];
#pragma unroll
    for (int u = 0; u < kXU; ++u) {
      const int kk = h0 + (wave * wsteps + u) * 32 + kg * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (u < wsteps && kk < H && tok_ok) v = *reinterpret_cast<const u32x4_t*>(xrow + kk);
      a[u] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      const int i = threadIdx.x + j * kThreads;
      if (i < np) {
        const int m = i < c4 ? 0 : 1, q = i - m * c4;
        const int f = 4 * q, r = f / N, n = f - r * N + m * N;  // row and first column of the piece
#pragma unroll
        for (int e = 0; e < 4; ++e) s_w[(n + e) * hcp + r] = wbuf[j][e];
      }
    }
    // what the pieces do not cover (an unaligned pointer, N % 4 != 0)
    for (int m = 0; m < (p.noisy ? 2 : 1); ++m) {
      const float* src = (m == 0 ? p.Wg : p.Wn) + static_cast<int64_t>(h0) * N;
      for (int i = 4 * c4 + threadIdx.x; i < cnt; i += kThreads) {
        const int r = i / N;
        s_w[(i - r * N + m * N) * hcp + r] = src[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kXU; ++u) {
      if (u < wsteps) {
        const int kl = (wave * wsteps + u) * 32 + kg * 8;  // K within the chunk
#pragma unroll
        for (int c = 0; c < NB16; ++c) {
          const int col = c * 16 + row;
          float wv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (col < n2) {
            const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(s_w + col * hcp + kl);
            const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(s_w + col * hcp + kl + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wv[e] = lo[e];
              wv[4 + e] = hi[e];
            }
            if (hn < hc) {  // rows past the chunk's end hold stale values
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (kl + e >= hn) wv[e] = 0.0f;
            }
          }
          bf16x8_t w1, w2, w3;
          split3(wv, w1, w2, w3);
          acc_hi[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], w1, acc_hi[c], 0, 0, 0);
          acc_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], w2, acc_lo[c], 0, 0, 0);
          acc_lo[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], w3, acc_lo[c], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one step's operands live at a time
    }
    __syncthreads();  // the chunk buffer is free again
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

hipError_t launch_router_mma(const RouterParams& p, hipStream_t s) {
  const int n2 = p.N * (p.noisy ? 2 : 1);
  const dim3 grid(static_cast<unsigned>((p.T + kTok - 1) / kTok));
#define MOE_ROUTER_MMA(NB) \
  hipLaunchKernelGGL(k_router_mma<NB>, grid, dim3(router_waves<NB>() * 64), 0, s, p, router_chunk_rows<NB>(p.H, n2))
  switch ((n2 + 15) / 16) {
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
