// Router on the matrix cores for bf16 activations.
//
// The router product x.W_g (and x.W_noise) is a skinny GEMM: T x H times
// H x N with N <= 64. Each fp32 router weight is split exactly into three
// bf16 parts, W = W1 + W2 + W3 (each part holds the next 8 significant bits;
// round-to-nearest-even leaves a remainder that the next part holds exactly),
// so every product x * W_i of a bf16 activation is exact in fp32 and
// v_mfma_f32_16x16x32_bf16 forms x.W with fp32 accumulation. The hi part and
// the two lower parts go to separate accumulators, and every sum covers a
// short run of H, which keeps the accumulated rounding error near that of a
// plain fp32 dot product.
//
// Two launches. k_router_part splits H into chunks: a block owns 64 or 128
// tokens and one chunk, each of its 8 waves a run of 32 to 128 rows of the
// chunk. A wave loads its rows' weights straight into the MFMA B-operand
// pattern (8 rows of one column per lane), splits them in registers and
// multiplies them with the x fragments of all the block's tokens; the 8
// waves' sums are added in wave order through LDS, and the chunk's partial
// logits go to the workspace. Every compute unit therefore splits only a
// chunk of the weights, not all of them. k_router_select adds a token's
// partials in chunk order and takes the routing decisions.
//
// The selection: one wave per token applies the noise term, KeepTopK and the
// gate of the chosen order: a lane's rank is the number of experts with a
// larger score, or an equal score and a lower index ("Llama 3 Meets MoE"
// review, section 3: ties to the lower expert index; a NaN score counts as
// -inf), and the experts of rank < k are kept in rank order (Mixtral:
// softmax over the kept scores; ST: softmax over all scores, section 5).
// Threads of the block then sum the per-expert counts, gate weights and
// softmax(logit) values over the block's 16 tokens in token order for the
// permutation and the balance statistics.
#include "common.h"
#include "kernels.h"

#include <algorithm>

typedef float f32x4_mma_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace moe {

namespace {

constexpr int kTok = 16;        // tokens per selection block (the permutation's histogram granularity)
constexpr int kPartWaves = 8;   // waves of a partial-product block
constexpr int kStepRows = 32;   // rows of H per MFMA step (the K of v_mfma_f32_16x16x32_bf16)

// token tiles of 16 per partial block: a wave's accumulators stay at 64
// registers for every column count
template <int NB16>
constexpr int part_tiles() { return 8 / NB16; }

// The partial-product grid: NB16 column tiles of 16 (1, 2, 4 or 8); KS MFMA
// steps per wave, so chunks of 256 * KS rows of H; token groups of
// 16 * part_tiles rows.
struct PartShape {
  int nb16, ks, chunk_rows, chunks, groups;
};
PartShape part_shape(int64_t T, int H, int N, int noisy) {
  PartShape s;
  const int n2 = N * (noisy ? 2 : 1);
  s.nb16 = n2 <= 16 ? 1 : (n2 <= 32 ? 2 : (n2 <= 64 ? 4 : 8));
  const int tb = 16 * (8 / s.nb16);
  s.groups = static_cast<int>((T + tb - 1) / tb);
  // nb16 steps per wave (at most 8 / nb16, for the weight registers): a
  // block then reads 64 KB of x (128 / nb16 tokens of 256 * nb16 rows), the
  // size that ran fastest at 8, 32 and 8 router columns over 4096 and 8192
  // tokens (measured against half and twice the chunk length)
  s.ks = std::min(s.nb16, 8 / s.nb16);
  s.chunk_rows = kPartWaves * kStepRows * s.ks;
  s.chunks = (H + s.chunk_rows - 1) / s.chunk_rows;
  return s;
}

// Exact three-way bf16 split of eight fp32 values, two at a time: the
// converts round to nearest even, and each remainder is exact in fp32.
__device__ __forceinline__ void split3(const float (&w)[8], bf16x8_t& p1, bf16x8_t& p2, bf16x8_t& p3) {
  u32x4_t q1, q2, q3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t v = {w[2 * i], w[2 * i + 1]};
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    const f32x2_t r1 = v - f32x2_t{__uint_as_float(h << 16), __uint_as_float(h & 0xffff0000u)};
    const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2_t));
    const f32x2_t r2 = r1 - f32x2_t{__uint_as_float(m << 16), __uint_as_float(m & 0xffff0000u)};
    q1[i] = h;
    q2[i] = m;
    q3[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2_t));
  }
  p1 = __builtin_bit_cast(bf16x8_t, q1);
  p2 = __builtin_bit_cast(bf16x8_t, q2);
  p3 = __builtin_bit_cast(bf16x8_t, q3);
}

__device__ __forceinline__ float lane_value(float v, int m) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), m));
}

// Partial logits of one chunk of H for one token group: part[chunk][t][c]
// = sum over the chunk's rows h of x[t][h] * W[h][c], W_g as columns [0, N)
// and W_noise as [N, 2N).
template <int NB16, int KS, bool NOISY>
__global__ __launch_bounds__(kPartWaves * 64) void k_router_part(RouterParams p) {
  constexpr int TT = part_tiles<NB16>();
  constexpr int TB = 16 * TT;
  constexpr int NC = 16 * NB16;
  constexpr int CR = kPartWaves * kStepRows * KS;
  __shared__ float s_red[kPartWaves][TB][NC];  // 64 KB

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, H = p.H;
  const int n2 = N * (NOISY ? 2 : 1);
  const int64_t T = p.T;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TB;
  const int chunk = blockIdx.y;
  const int tv = static_cast<int>(T - tok0 < TB ? T - tok0 : TB);  // tokens of this block
  const int h0 = chunk * CR + wave * (kStepRows * KS);                // this wave's first row of H

  // MFMA roles: A row / B column `row`, K group `kg` (rows 8 kg .. 8 kg + 7
  // of the step)
  const int row = lane & 15, kg = lane >> 4;
  // x rows of this block through a buffer descriptor: a load past the rows
  // or past H (offset kOOB) returns zeros
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
  const __amdgpu_buffer_rsrc_t rx = uniform_rsrc(x + tok0 * H, static_cast<int64_t>(tv) * H * 2);
  bf16x8_t a[KS][TT];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int kk = h0 + s * kStepRows + 8 * kg, tr = 16 * t + row;
      const uint32_t off = (kk < H && tr < tv) ? static_cast<uint32_t>(tr * H + kk) * 2u : kOOB;
      a[s][t] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
  // the weights in the B pattern: lane (row, kg) of column tile c takes
  // column 16 c + row at the step's rows 8 kg .. 8 kg + 7. A lane's column
  // lies in W_g or in W_noise: each matrix is read through its own
  // descriptor, the other load's offset is out of range and reads zero, as
  // do columns past n2 and rows past H.
  const int64_t w_bytes = static_cast<int64_t>(H) * N * 4;
  const __amdgpu_buffer_rsrc_t rg = uniform_rsrc(p.Wg, w_bytes);
  const __amdgpu_buffer_rsrc_t rn = uniform_rsrc(NOISY ? p.Wn : p.Wg, w_bytes);
  float wv[KS][NB16][8];
#pragma unroll
  for (int c = 0; c < NB16; ++c) {
    const int col = 16 * c + row;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int h = h0 + s * kStepRows + 8 * kg + e;
        const uint32_t og = (col < N && h < H) ? static_cast<uint32_t>(h * N + col) * 4u : kOOB;
        wv[s][c][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, og, 0, 0));
      }
  }
  if (NOISY) {
#pragma unroll
    for (int c = 0; c < NB16; ++c) {
      const int col = 16 * c + row;
      const bool in_n = col >= N && col < n2;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int h = h0 + s * kStepRows + 8 * kg + e;
          const uint32_t on = (in_n && h < H) ? static_cast<uint32_t>(h * N + col - N) * 4u : kOOB;
          wv[s][c][e] += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, on, 0, 0));
        }
    }
  }

  f32x4_mma_t acc_hi[TT][NB16], acc_lo[TT][NB16];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < NB16; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_hi[t][c][r] = acc_lo[t][c][r] = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int c = 0; c < NB16; ++c) {
      bf16x8_t w1, w2, w3;
      split3(wv[s][c], w1, w2, w3);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        acc_hi[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][t], w1, acc_hi[t][c], 0, 0, 0);
        acc_lo[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][t], w2, acc_lo[t][c], 0, 0, 0);
        acc_lo[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s][t], w3, acc_lo[t][c], 0, 0, 0);
      }
    }

  // lane holds output rows 4 kg + r and column `row` of each product; the
  // waves' sums are added in wave order
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < NB16; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_red[wave][16 * t + 4 * kg + r][16 * c + row] = acc_hi[t][c][r] + acc_lo[t][c][r];
  __syncthreads();
  float* __restrict__ dst = p.part + (static_cast<int64_t>(chunk) * T + tok0) * n2;
  for (int i = threadIdx.x; i < tv * n2; i += kPartWaves * 64) {
    const int t = i / n2, c = i - t * n2;
    float v = s_red[0][t][c];
#pragma unroll
    for (int w = 1; w < kPartWaves; ++w) v += s_red[w][t][c];
    dst[i] = v;
  }
}

// Sums of the chunks' partial logits in chunk order, then the noise term,
// KeepTopK, the gates and the block's statistics, for 16 tokens per block.
// A token takes a group of NM lanes (NM >= N, a power of two), lane e of the
// group holding expert e, so a wave holds 64 / NM tokens; the experts'
// values move within a group by lane shuffles. Every load is requested up
// front (out-of-range offsets read zero), every lane runs the same
// instructions (a token past the batch computes on zeros and stores
// nothing), and every global store comes after the block's last barrier.
template <int NM>
__global__ __launch_bounds__(NM / 4 * 64) void k_router_select(RouterParams p, int chunks) {
  constexpr int kTPW = 64 / NM;  // tokens per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = lane & ~(NM - 1), e = lane & (NM - 1);  // the group's first lane; this lane's expert
  const int t = wave * kTPW + base / NM;                   // this group's token within the block
  const int N = p.N, k = p.k;
  const int n2 = N * (p.noisy ? 2 : 1);
  const int64_t T = p.T;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int tv = static_cast<int>(T - tok0 < kTok ? T - tok0 : kTok);
  const bool live = t < tv;
  const bool valid = e < N;
  const int64_t g = tok0 + t;
  const uint64_t gmask = NM == 64 ? ~0ull : ((1ull << NM) - 1) << base;
  // the lowest lane of this group where pred holds (one must)
  auto first = [&](bool pred) { return static_cast<int>(__builtin_ctzll(__ballot(pred) & gmask)); };

  // the noise draw and the partial logits of expert e (column e of W_g,
  // column N + e of W_noise), sixteen chunks' worth at a time
  const __amdgpu_buffer_rsrc_t re = uniform_rsrc(p.noisy ? p.eps : p.part, p.noisy ? T * N * 4 : 0);
  const float epsv = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 re, (p.noisy && valid && live) ? static_cast<uint32_t>(g * N + e) * 4u : kOOB, 0, 0));
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(p.part, static_cast<int64_t>(chunks) * T * n2 * 4);
  const uint32_t cs = static_cast<uint32_t>(T * n2) * 4u;  // bytes of one chunk's partials
  const bool lok = valid && live, nok = p.noisy && valid && live;
  const uint32_t ol = static_cast<uint32_t>(g * n2 + e) * 4u, on = ol + static_cast<uint32_t>(N) * 4u;
  float lv = 0.0f, nv = 0.0f;
  for (int ch0 = 0; ch0 < chunks; ch0 += 16) {
    float ql[16], qn[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool c_ok = ch0 + j < chunks;
      const uint32_t co = static_cast<uint32_t>(ch0 + j) * cs;
      ql[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (c_ok && lok) ? co + ol : kOOB, 0, 0));
      qn[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, (c_ok && nok) ? co + on : kOOB, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      lv += ql[j];
      nv += qn[j];
    }
  }

  if (!valid) lv = -INFINITY;
  float hv = lv;
  // H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i), the
  // normal draw being the input eps[t, i]
  const float sp = (p.noisy && valid) ? softplus(nv) : 1.0f;
  if (p.noisy && valid) hv = fmaf(epsv, sp, lv);
  // a NaN score counts as -inf in KeepTopK and the gates, so the rank below
  // is a strict total order and exactly k experts are kept
  if (hv != hv) hv = -INFINITY;
  // rank: experts with a larger score, or an equal one at a lower index
  int rank = 0;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float sm = __shfl(hv, base + m);
    if (m < N) rank += (sm > hv || (sm == hv && m < e)) ? 1 : 0;
  }
  const bool kept = valid && rank < k;
  const float hmax = __shfl(hv, first(valid && rank == 0));
  // Mixtral order: softmax over the kept scores; ST: over all N scores.
  // The denominator adds the terms in expert order.
  const float ex = (p.order == 0 ? kept : valid) ? expf(hv - hmax) : 0.0f;
  float den = 0.0f;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const float v = __shfl(ex, base + m);
    if (m < N) den += v;
  }
  const float wgt = kept ? ex / den : 0.0f;
  float pv = 0.0f, slv = 0.0f;
  if (p.stat_part) {
    float lmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const float v = __shfl(lv, base + m);
      if (m < N) lmax = fmaxf(lmax, v);
    }
    const float el = valid ? expf(lv - lmax) : 0.0f;
    float ls = 0.0f;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const float v = __shfl(el, base + m);
      if (m < N) ls += v;
    }
    pv = el / ls;
    if (p.smooth) {
      // smooth load (Shazeer et al. 2017, the TopK Noisy Gate the LLaMA-MoE
      // hub page names): the chance that expert i stays in the top k when
      // only its own draw is taken again, Phi((clean logit - k-th highest
      // other score) / Softplus(noise logit)); the k-th highest other score
      // is the score of rank k for a kept expert, of rank k - 1 otherwise
      // (-inf when no expert has rank k)
      const float v1 = __shfl(hv, first(valid && rank == k - 1));
      const bool has_k = (__ballot(valid && rank == k) & gmask) != 0;
      const float v2 = has_k ? __shfl(hv, first(valid && rank == k)) : -INFINITY;
      const float z = (lv - (kept ? v2 : v1)) / sp;
      slv = valid ? 0.5f * erfcf(z * -0.70710678118654752f) : 0.0f;
    }
  }
  // tokens past the batch and lanes past N add zeros to the block's sums
  __shared__ float s_sel[kTok][NM];  // gate weight of expert e if kept, else 0
  __shared__ int s_take[kTok][NM];   // 1 if expert e is among the token's top k
  __shared__ float s_p[kTok][NM];    // softmax of the clean logits
  __shared__ float s_sl[kTok][NM];   // smooth-load probability of expert e
  s_take[t][e] = (live && kept) ? 1 : 0;
  s_sel[t][e] = live ? wgt : 0.0f;
  s_p[t][e] = live ? pv : 0.0f;
  s_sl[t][e] = live ? slv : 0.0f;
  __syncthreads();

  if (live && valid) {
    if (p.logits) p.logits[g * N + e] = lv;
    if (p.noise_logits && p.noisy) p.noise_logits[g * N + e] = nv;
    if (kept) {
      p.topk_idx[g * k + rank] = e;
      p.topk_w[g * k + rank] = wgt;
    }
  }
  // per-block sums over the tokens, in token order
  if (p.hist && threadIdx.x < N) {
    const int n = threadIdx.x;
    int cnt = 0;
    float imp = 0.0f, ps = 0.0f, sl = 0.0f;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      cnt += s_take[u][n];
      imp += s_sel[u][n];
      ps += s_p[u][n];
      sl += s_sl[u][n];
    }
    p.hist[static_cast<int64_t>(blockIdx.x) * N + n] = cnt;
    if (p.stat_part) {
      float* part = p.stat_part + (static_cast<int64_t>(blockIdx.x) * N + n) * kStatsPerExpert;
      part[0] = imp;
      part[1] = ps;
      part[2] = sl;
    }
  }
}

}  // namespace

int64_t router_part_floats(int64_t T, int H, int N, int noisy) {
  const PartShape sh = part_shape(T, H, N, noisy);
  return static_cast<int64_t>(sh.chunks) * T * N * (noisy ? 2 : 1);
}

hipError_t launch_router_mma(const RouterParams& p, hipStream_t s) {
  const PartShape sh = part_shape(p.T, p.H, p.N, p.noisy);
  const dim3 grid(static_cast<unsigned>(sh.groups), static_cast<unsigned>(sh.chunks)), block(kPartWaves * 64);
#define MOE_ROUTER_PART(NB, KS)                                                    \
  do {                                                                             \
    if (p.noisy)                                                                   \
      hipLaunchKernelGGL((k_router_part<NB, KS, true>), grid, block, 0, s, p);     \
    else                                                                           \
      hipLaunchKernelGGL((k_router_part<NB, KS, false>), grid, block, 0, s, p);    \
  } while (0)
  switch (sh.nb16) {  // steps per wave: part_shape's choice for each column count
    case 1: MOE_ROUTER_PART(1, 1); break;
    case 2: MOE_ROUTER_PART(2, 2); break;
    case 4: MOE_ROUTER_PART(4, 2); break;
    default: MOE_ROUTER_PART(8, 1); break;
  }
#undef MOE_ROUTER_PART
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sgrid(static_cast<unsigned>((p.T + kTok - 1) / kTok));
#define MOE_ROUTER_SELECT(NM) hipLaunchKernelGGL(k_router_select<NM>, sgrid, dim3(NM / 4 * 64), 0, s, p, sh.chunks)
  if (p.N <= 4)
    MOE_ROUTER_SELECT(4);
  else if (p.N <= 8)
    MOE_ROUTER_SELECT(8);
  else if (p.N <= 16)
    MOE_ROUTER_SELECT(16);
  else if (p.N <= 32)
    MOE_ROUTER_SELECT(32);
  else
    MOE_ROUTER_SELECT(64);
#undef MOE_ROUTER_SELECT
  return hipGetLastError();
}

}  // namespace moe
