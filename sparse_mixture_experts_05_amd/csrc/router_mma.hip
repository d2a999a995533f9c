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
// A block owns 16 tokens and walks H in chunks through two LDS buffers: while
// the waves split and multiply chunk c, the fp32 weight rows and x of chunk
// c + 1 are in flight, and they are written to the other buffer (transposed,
// so that a lane reads its eight operand values of one column with two
// 16-byte reads) before the barrier that ends the chunk.
//
// With at most 8 router columns, half the 16 columns of the MFMA B operand
// would be zero, so they are "folded": columns 8..15 carry the same 8 router
// columns for the next 32 rows of H, and the A rows 8..15 carry the same 8
// tokens at those rows. The diagonal 8 x 8 blocks of the product are the two
// halves of the dot products; the off-diagonal blocks are not used. Every
// lane then splits weight values that are used, which halves the splitting
// work per row of H.
//
// After the product, one wave per token applies the noise term, KeepTopK and
// the gate of the chosen order: a lane's rank is the number of experts with a
// larger score, or an equal score and a lower index ("Llama 3 Meets MoE"
// review, section 3: ties to the lower expert index; a NaN score counts as
// -inf), and the experts of rank < k are kept in rank order (Mixtral:
// softmax over the kept scores; ST: softmax over all scores, section 5). Threads of the block then sum the
// per-expert counts, gate weights and softmax(logit) values over the block's
// tokens in token order for the permutation and the balance statistics.
#include "common.h"
#include "kernels.h"

#include <algorithm>

typedef float f32x4_mma_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace moe {

namespace {

constexpr int kTok = 16;  // tokens per block (M of the MFMA)
// waves per block, each over 1/W of a chunk's rows: more waves for fewer
// output columns, fewer when the partial sums of every wave would not fit
template <int NB16>
constexpr int router_waves() { return NB16 <= 2 ? 16 : (NB16 <= 4 ? 8 : 4); }

constexpr int kWFloats = 16 * 1024;  // fp32 weights of one chunk (64 KB); two buffers
constexpr int kWPad = 4;             // floats of padding per LDS column
constexpr int kWBuf = kWFloats + kWPad * 128;  // one buffer, up to 128 padded columns

// 16-byte x loads per lane per chunk (two chunks stay in registers): folded
// chunks give a wave two steps of two A fragments; otherwise the buffer holds
// at most two steps per wave
template <bool FOLD>
constexpr int router_xl() { return FOLD ? 4 : 2; }

// Rows of H one MFMA step covers: 32, or 64 when the columns are folded.
template <bool FOLD>
constexpr int unit_rows() { return FOLD ? 64 : 32; }

// Rows of H per chunk: whole steps for every wave, within one buffer for all
// n2 columns and within the lanes' x registers.
template <int NB16, bool FOLD>
int router_chunk_rows(int H, int n2) {
  const int unit = unit_rows<FOLD>() * router_waves<NB16>();
  const int max_units = FOLD ? router_xl<FOLD>() / 2 : router_xl<FOLD>();
  int rows = kWFloats / n2 / unit * unit;
  rows = std::min(rows, max_units * unit);
  rows = std::max(rows, unit);
  return std::min(rows, (H + unit - 1) / unit * unit);
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

// SHORT: H fits in the two buffers; the weights are staged first, then all
// of x is requested at once.
template <int NB16, bool FOLD, bool SHORT>
__global__ __launch_bounds__(router_waves<NB16>() * 64) void k_router_mma(RouterParams p, int hc) {
  constexpr int kWaves = router_waves<NB16>();
  constexpr int kThreads = kWaves * 64;
  constexpr int NC = NB16 * 16;
  constexpr int kXL = router_xl<FOLD>();
  constexpr int UR = unit_rows<FOLD>();
  constexpr int AF = FOLD ? 2 : 1;        // A fragments per step (token halves when folded)
  constexpr int kU = kXL / AF;            // most steps of one wave in one chunk
  constexpr int kP = kWFloats / 4 / kThreads;  // most 16-byte weight pieces per thread per chunk
  static_assert(!FOLD || NB16 == 1, "folding is for at most 8 columns");
  // the weight chunks; after the product, the per-wave partial sums
  __shared__ __attribute__((aligned(16))) float s_w[2 * kWBuf];
  static_assert(kWaves * kTok * NC <= 2 * kWBuf, "partials fit in the weight buffers");
  __shared__ float s_log[kTok][NC];  // clean logits, then noise logits

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = p.N, H = p.H, k = p.k;
  const int64_t T = p.T;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const uint16_t* __restrict__ x = static_cast<const uint16_t*>(p.x);
  const int n2 = N * (p.noisy ? 2 : 1);  // real columns; the padding stays zero

  // MFMA roles: A row / B column `row`, K group `kg` (8 of the step's rows).
  // Folded, row bit 3 selects the upper 32 rows of the 64-row step on both
  // sides, and A row r of token half th is token 8 * th + (r & 7).
  const int row = lane & 15, kg = lane >> 4;
  const int koff = FOLD ? 32 * (row >> 3) + 8 * kg : 8 * kg;
  const int bcol = FOLD ? (row & 7) : row;
  // x rows of this block through a buffer descriptor: a load past the rows
  // or past H (offset kOOB) returns zeros, so every lane issues the same loads
  // in every chunk and the waits for them are exact
  const int tv = static_cast<int>(T - tok0 < kTok ? T - tok0 : kTok);  // tokens of this block
  const __amdgpu_buffer_rsrc_t rx = uniform_rsrc(x + tok0 * H, static_cast<int64_t>(tv) * H * 2);
  int trow[AF];
#pragma unroll
  for (int th = 0; th < AF; ++th) trow[th] = FOLD ? 8 * th + (row & 7) : row;
  // f / N for the weight pieces' rows: a multiply-high by ceil(2^32 / N),
  // exact for f < 2^32 / N (f stays below a chunk's hc * N floats); N = 1,
  // whose multiplier does not fit 32 bits, is the identity
  const uint32_t n_inv = N > 1 ? 0xFFFFFFFFu / static_cast<uint32_t>(N) + 1u : 0u;
  auto div_n = [&](int f) { return N > 1 ? static_cast<int>(__umulhi(static_cast<uint32_t>(f), n_inv)) : f; };
  // the noise draws of this wave's tokens, requested now so that their
  // latency hides behind the product
  constexpr int kTW = (kTok + kWaves - 1) / kWaves;  // tokens per wave in the gate step
  float eps_pre[kTW];
#pragma unroll
  for (int i = 0; i < kTW; ++i) {
    const int t = wave + i * kWaves;
    eps_pre[i] = (p.noisy && lane < N && t < kTok && tok0 + t < T) ? p.eps[(tok0 + t) * N + lane] : 0.0f;
  }
  const int wu = hc / UR / kWaves;  // this wave's steps per chunk
  const int hcp = hc + kWPad;       // LDS column stride: column j holds the chunk's rows contiguous

  f32x4_mma_t acc_hi[NB16][AF], acc_lo[NB16][AF];
#pragma unroll
  for (int c = 0; c < NB16; ++c)
#pragma unroll
    for (int th = 0; th < AF; ++th)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_hi[c][th][r] = acc_lo[c][th][r] = 0.0f;

  // 16-byte weight loads need aligned pointers and whole rows per piece
  const bool vec = (reinterpret_cast<uintptr_t>(p.Wg) & 15) == 0 &&
                   (!p.noisy || (reinterpret_cast<uintptr_t>(p.Wn) & 15) == 0) && N % 4 == 0;
  const int64_t w_bytes = static_cast<int64_t>(H) * N * 4;
  const __amdgpu_buffer_rsrc_t rw[2] = {uniform_rsrc(p.Wg, w_bytes), uniform_rsrc(p.noisy ? p.Wn : p.Wg, w_bytes)};
  // weight piece j of this thread: matrix (W_g, or W_noise for the upper half
  // of the pieces when noisy) and 16-byte piece index within the chunk
  auto piece = [&](int j, int& m, int& q) {
    m = (p.noisy && j >= kP / 2) ? 1 : 0;
    q = threadIdx.x + (j - m * (kP / 2)) * kThreads;
  };

  f32x4_t wbuf[kP], wbuf2[kP];
  bf16x8_t a_cur[kXL], a_nxt[kXL];  // x of this chunk and of the next
  // a chunk's weight rows, W_g as columns [0, N) and W_noise as [N, 2N), in
  // 16-byte pieces
  auto load_w = [&](int h0, f32x4_t (&wb)[kP]) {
    const int hn = min(hc, H - h0);
    const int c4 = vec ? hn * N / 4 : 0;
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      int m, q;
      piece(j, m, q);
      const uint32_t off = q < c4 ? static_cast<uint32_t>(h0 * N + 4 * q) * 4u : kOOB;
      wb[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw[m], off, 0, 0));
    }
  };
  auto load_x = [&](int h0, bf16x8_t (&a)[kXL]) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int th = 0; th < AF; ++th) {
        const int kk = h0 + (wave * wu + u) * UR + koff;
        const bool ok = u < wu && kk < H && trow[th] < tv;
        const uint32_t off = ok ? static_cast<uint32_t>(trow[th] * H + kk) * 2u : kOOB;
        a[u * AF + th] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      }
  };
  // transposed stores of the pieces, and what they do not cover (an
  // unaligned pointer, N % 4 != 0) straight from global memory
  auto store_w = [&](int h0, float* sb, const f32x4_t (&wb)[kP]) {
    const int hn = min(hc, H - h0);
    const int cnt = hn * N, c4 = vec ? cnt / 4 : 0;
#pragma unroll
    for (int j = 0; j < kP; ++j) {
      int m, q;
      piece(j, m, q);
      if (q < c4) {
        const int f = 4 * q, r = div_n(f), n = f - r * N + m * N;  // row and first column of the piece
#pragma unroll
        for (int e = 0; e < 4; ++e) sb[(n + e) * hcp + r] = wb[j][e];
      }
    }
    for (int m = 0; m < (p.noisy ? 2 : 1); ++m) {
      const float* src = (m == 0 ? p.Wg : p.Wn) + static_cast<int64_t>(h0) * N;
      for (int i = 4 * c4 + threadIdx.x; i < cnt; i += kThreads) {
        const int r = div_n(i);
        sb[(i - r * N + m * N) * hcp + r] = src[i];
      }
    }
  };
  auto compute = [&](int h0, const float* sb, const bf16x8_t (&a)[kXL]) {
    const int hn = min(hc, H - h0);  // weight rows in this chunk; the rest hold stale values
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u < wu) {
        const int kl = (wave * wu + u) * UR + koff;  // row within the chunk
#pragma unroll
        for (int c = 0; c < NB16; ++c) {
          const int col = c * 16 + bcol;
          float wv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (col < n2) {
            // col * hcp + kl is a multiple of 4 floats
            const f32x4_t* src = reinterpret_cast<const f32x4_t*>(sb) + ((col * hcp + kl) >> 2);
            const f32x4_t lo = src[0], hi = src[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wv[e] = lo[e];
              wv[4 + e] = hi[e];
            }
            if (hn < hc) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (kl + e >= hn) wv[e] = 0.0f;
            }
          }
          bf16x8_t w1, w2, w3;
          split3(wv, w1, w2, w3);
#pragma unroll
          for (int th = 0; th < AF; ++th) {
            const bf16x8_t af = a[u * AF + th];
            acc_hi[c][th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, w1, acc_hi[c][th], 0, 0, 0);
            acc_lo[c][th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, w2, acc_lo[c][th], 0, 0, 0);
            acc_lo[c][th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, w3, acc_lo[c][th], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one step's operands live at a time
    }
  };

  if constexpr (SHORT) {
    // Both chunks' weights are requested first and stored; x follows. Every
    // block reads the same weights, and their first reads from memory would
    // otherwise queue behind the whole of x.
    load_w(0, wbuf);
    load_w(hc, wbuf2);
    store_w(0, s_w, wbuf);
    store_w(hc, s_w + kWBuf, wbuf2);
    __syncthreads();
    load_x(0, a_cur);
    load_x(hc, a_nxt);
    compute(0, s_w, a_cur);
    if (hc < H) compute(hc, s_w + kWBuf, a_nxt);
    __syncthreads();
  } else {
    // software pipeline over the chunks: chunk c + 1 loads while chunk c
    // computes, and is stored to the other buffer before the barrier that
    // ends chunk c
    load_w(0, wbuf);
    load_x(0, a_cur);
    store_w(0, s_w, wbuf);
    // chunk 0's x has landed too: no load is pending where the loop starts,
    // so the waits inside it count only the next chunk's loads
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int h0 = 0, c = 0; h0 < H; h0 += hc, ++c) {
      const bool more = h0 + hc < H;
      if (more) {
        load_w(h0 + hc, wbuf);
        load_x(h0 + hc, a_nxt);
      }
      compute(h0, s_w + (c & 1) * kWBuf, a_cur);
      if (more) store_w(h0 + hc, s_w + ((c + 1) & 1) * kWBuf, wbuf);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kXL; ++i) a_cur[i] = a_nxt[i];
    }
  }

  // lane holds output rows 4 * kg + r and column `row` of each product
  if constexpr (FOLD) {
    // the diagonal blocks: rows 0..7 x columns 0..7 (lower 32 rows of each
    // step) and rows 8..15 x columns 8..15 (upper 32 rows)
    float (*s_part)[2][kTok][8] = reinterpret_cast<float (*)[2][kTok][8]>(s_w);
    const int half = kg >> 1;
    if (half == (row >> 3)) {
#pragma unroll
      for (int th = 0; th < AF; ++th)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_part[wave][half][8 * th + ((4 * kg + r) & 7)][row & 7] = acc_hi[0][th][r] + acc_lo[0][th][r];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTok * 8; i += kThreads) {
      const int t = i / 8, c = i % 8;
      float v = s_part[0][0][t][c] + s_part[0][1][t][c];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_part[w][0][t][c] + s_part[w][1][t][c];
      s_log[t][c] = v;
    }
  } else {
    float (*s_part)[kTok][NC] = reinterpret_cast<float (*)[kTok][NC]>(s_w);
#pragma unroll
    for (int c = 0; c < NB16; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_part[wave][kg * 4 + r][c * 16 + row] = acc_hi[c][0][r] + acc_lo[c][0][r];
    __syncthreads();
    for (int i = threadIdx.x; i < kTok * NC; i += kThreads) {
      const int t = i / NC, c = i % NC;
      float v = s_part[0][t][c];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += s_part[w][t][c];
      s_log[t][c] = v;
    }
  }
  __syncthreads();

  // one wave per token, lane n holding expert n: noise, KeepTopK, gates
  __shared__ float s_sel[kTok][64];  // gate weight of expert n if kept, else 0
  __shared__ int s_take[kTok][64];   // 1 if expert n is among the token's top k
  __shared__ float s_p[kTok][64];    // softmax of the clean logits
  __shared__ float s_sl[kTok][64];   // smooth-load probability of expert n
  const bool valid = lane < N;
#pragma unroll
  for (int i = 0; i < kTW; ++i) {
    const int t = wave + i * kWaves;
    const int64_t g = tok0 + t;
    if (t >= kTok || g >= T) break;  // wave-uniform
    const float lv = valid ? s_log[t][lane] : -INFINITY;
    float hv = lv;
    // H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i), the
    // normal draw being the input eps[t, i]
    const float sp = (p.noisy && valid) ? softplus(s_log[t][N + lane]) : 1.0f;
    if (p.noisy && valid) hv = fmaf(eps_pre[i], sp, lv);
    // a NaN score counts as -inf in KeepTopK and the gates, so the rank below
    // is a strict total order and exactly k experts are kept
    if (hv != hv) hv = -INFINITY;
    if (p.logits && valid) p.logits[g * N + lane] = lv;
    if (p.noise_logits && p.noisy && valid) p.noise_logits[g * N + lane] = s_log[t][N + lane];
    // rank: experts with a larger score, or an equal one at a lower index
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const float sm = lane_value(hv, m);
      rank += (sm > hv || (sm == hv && m < lane)) ? 1 : 0;
    }
    const bool kept = valid && rank < k;
    const float hmax = lane_value(hv, static_cast<int>(__builtin_ctzll(__ballot(valid && rank == 0))));
    // Mixtral order: softmax over the kept scores; ST: over all N scores.
    // The denominator adds the terms in expert order.
    const float ex = (p.order == 0 ? kept : valid) ? expf(hv - hmax) : 0.0f;
    float den = 0.0f;
    for (int m = 0; m < N; ++m) den += lane_value(ex, m);
    const float wgt = kept ? ex / den : 0.0f;
    if (kept) {
      p.topk_idx[g * k + rank] = lane;
      p.topk_w[g * k + rank] = wgt;
    }
    s_take[t][lane] = kept ? 1 : 0;
    s_sel[t][lane] = wgt;
    if (p.stat_part) {
      float lmax = -INFINITY;
      for (int m = 0; m < N; ++m) lmax = fmaxf(lmax, lane_value(lv, m));
      const float el = valid ? expf(lv - lmax) : 0.0f;
      float ls = 0.0f;
      for (int m = 0; m < N; ++m) ls += lane_value(el, m);
      s_p[t][lane] = el / ls;
      if (p.smooth) {
        // smooth load (Shazeer et al. 2017, the TopK Noisy Gate the LLaMA-MoE
        // hub page names): the chance that expert i stays in the top k when
        // only its own draw is taken again, Phi((clean logit - k-th highest
        // other score) / Softplus(noise logit)); the k-th highest other score
        // is the score of rank k for a kept expert, of rank k - 1 otherwise
        // (-inf when no expert has rank k)
        const uint64_t bk1 = __ballot(valid && rank == k - 1), bk = __ballot(valid && rank == k);
        const float v1 = lane_value(hv, static_cast<int>(__builtin_ctzll(bk1)));
        const float v2 = bk ? lane_value(hv, static_cast<int>(__builtin_ctzll(bk))) : -INFINITY;
        const float z = (lv - (kept ? v2 : v1)) / sp;
        s_sl[t][lane] = valid ? 0.5f * erfcf(z * -0.70710678118654752f) : 0.0f;
      }
    }
  }
  __syncthreads();

  // per-block sums over the tokens, in token order
  if (p.hist && threadIdx.x < N) {
    const int n = threadIdx.x;
    int cnt = 0;
    float imp = 0.0f, ps = 0.0f, sl = 0.0f;
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      const bool ok = t < tv;
      cnt += ok ? s_take[t][n] : 0;
      imp += ok ? s_sel[t][n] : 0.0f;
      ps += ok ? s_p[t][n] : 0.0f;
      sl += (ok && p.smooth) ? s_sl[t][n] : 0.0f;
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

hipError_t launch_router_mma(const RouterParams& p, hipStream_t s) {
  const int n2 = p.N * (p.noisy ? 2 : 1);
  const dim3 grid(static_cast<unsigned>((p.T + kTok - 1) / kTok));
#define MOE_ROUTER_MMA(NB, FOLD, SHORT)                                                                \
  do {                                                                                                 \
    const int hc = router_chunk_rows<NB, FOLD>(p.H, n2);                                               \
    if (SHORT && 2 * hc >= p.H)                                                                        \
      hipLaunchKernelGGL((k_router_mma<NB, FOLD, SHORT>), grid, dim3(router_waves<NB>() * 64), 0, s, p, hc); \
    else                                                                                               \
      hipLaunchKernelGGL((k_router_mma<NB, FOLD, false>), grid, dim3(router_waves<NB>() * 64), 0, s, p, hc); \
  } while (0)
  switch ((n2 + 15) / 16) {
    case 1:
      if (n2 <= 8) MOE_ROUTER_MMA(1, true, true);
      else MOE_ROUTER_MMA(1, false, true);
      break;
    case 2: MOE_ROUTER_MMA(2, false, true); break;
    case 3: MOE_ROUTER_MMA(3, false, false); break;
    case 4: MOE_ROUTER_MMA(4, false, false); break;
    case 5: MOE_ROUTER_MMA(5, false, false); break;
    case 6: MOE_ROUTER_MMA(6, false, false); break;
    case 7: MOE_ROUTER_MMA(7, false, false); break;
    default: MOE_ROUTER_MMA(8, false, false); break;
  }
#undef MOE_ROUTER_MMA
  return hipGetLastError();
}

}  // namespace moe
