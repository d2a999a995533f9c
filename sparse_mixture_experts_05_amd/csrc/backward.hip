// Backward of the MoE layer on gfx950, for a training step (continual
// pre-training is the pages' main workload: LLaMA-MoE hub page and paper
// summary; the balance loss comes from the LLaMA-MoE v2 article's gating
// section). Gradients of L = <dy, y> + d_balance * balance; KeepTopK and the
// capacity clip are piecewise constant, so the router gets gradient only
// through the chosen experts' gate weights.
//
// The kernels here move and reduce data; the four expert GEMMs of the
// backward (dh = dE Wdown, dx = dg Wgate + du Wup, and the weight gradients)
// run on the matrix-core tiles of gemm_mfma.hip, which read the operands whose
// rows are K rows (the weights, and every operand of the weight gradients) in
// place, through gfx950's transposing LDS reads.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// Cache policy of the loads of data a launch reads exactly once and that no
// later launch of the step reads again (dy, y_perm and dx_perm rows): the nt
// bit, as for the stores of dx.
constexpr int kReadOnce = 2;

__device__ __forceinline__ float lane_value(float v, int m) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), m));
}

// Sum over the 256 threads of a block in a fixed order (each wave's butterfly,
// then the four waves in order); every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// The gate weights' gradients (s_dw, per slot) back to the router logits:
// the block's first wave, lane n holding expert n.
__device__ __forceinline__ void gate_to_logits(const BwdGateParams& p, int64_t t, const float* s_dw) {
  const int k = p.k, N = p.N;
  const int lane = threadIdx.x;
  const bool valid = lane < N;
  // this lane's expert among the token's top k (the slot index j), if any
  int jj = -1;
  for (int j = 0; j < k; ++j)
    if (p.topk_idx[t * k + j] == lane) jj = j;
  const float dw = jj >= 0 ? s_dw[jj] : 0.0f;
  float dH = 0.0f;
  const float lv = valid ? p.logits[t * N + lane] : -INFINITY;
  float spv = 0.0f, nz = 0.0f, ev = 0.0f;
  if (p.noisy && valid) {
    nz = p.noise_logits[t * N + lane];
    ev = p.eps[t * N + lane];
    spv = softplus(nz);
  }
  if (p.order == 0) {
    const float wv = jj >= 0 ? p.topk_w[t * k + jj] : 0.0f;
    float sdot = 0.0f;
    for (int j = 0; j < k; ++j) sdot += p.topk_w[t * k + j] * s_dw[j];
    dH = jj >= 0 ? wv * (dw - sdot) : 0.0f;
  } else {
    // the router's scores and softmax, recomputed with the same operations
    float hv = lv;
    if (p.noisy && valid) hv = fmaf(ev, spv, lv);
    if (hv != hv) hv = -INFINITY;
    const float hmax = lane_value(hv, p.topk_idx[t * k]);
    const float ex = valid ? expf(hv - hmax) : 0.0f;
    float den = 0.0f;
    for (int m = 0; m < N; ++m) den += lane_value(ex, m);
    const float pv = ex / den;
    float sdot = 0.0f;
    const float pd = pv * dw;
    for (int m = 0; m < N; ++m) sdot += lane_value(pd, m);
    dH = valid ? pv * (dw - sdot) : 0.0f;
  }
  float dl = dH;
  if (p.d_balance != 0.0f) {
    float lmax = -INFINITY;
    for (int m = 0; m < N; ++m) lmax = fmaxf(lmax, lane_value(lv, m));
    const float el = valid ? expf(lv - lmax) : 0.0f;
    float ls = 0.0f;
    for (int m = 0; m < N; ++m) ls += lane_value(el, m);
    const float pc = el / ls;
    const float fv = valid ? static_cast<float>(p.counts[lane]) / (static_cast<float>(p.T) * k) : 0.0f;
    const float fpc = fv * pc;
    float fp = 0.0f;
    for (int m = 0; m < N; ++m) fp += lane_value(fpc, m);
    dl += p.d_balance / static_cast<float>(p.T) * pc * (fv - fp);
  }
  if (valid) {
    p.dlog[t * N + lane] = dl;
    if (p.noisy) p.dnz[t * N + lane] = dH * ev * __builtin_amdgcn_rcpf(1.0f + expf(-nz));
  }
}

// One token per block: dw_j = s <dy_t, E_j> over the kept slots (E_j is the
// y_perm row of slot j), dE_j = bf16(s w_j dy_t) into the slot's row, then one
// wave takes the gate weights back to the scores and the router logits:
//   Mixtral (softmax over the kept scores): dH = w_j (dw_j - sum w dw) at idx_j;
//   ST (softmax over all scores): dH = p (dp - <p, dp>), dp = dw at idx_j;
//   balance: dlogit += d_balance / T * p_clean (f - <f, p_clean>), f = load/(T k);
//   noise: dn = dH * eps * sigmoid(noise logit).
template <int KM>  // k <= KM
__global__ __launch_bounds__(256) void k_bwd_gate(BwdGateParams p) {
  __shared__ float red[4][KM];
  __shared__ float s_dw[64];
  const int64_t t = blockIdx.x;
  if (t == 0 && p.zero)
    for (int i = threadIdx.x; i < p.zero_n; i += 256) p.zero[i] = 0;
  const int H = p.H, k = p.k, N = p.N;
  const float s = p.scale;
  // the token's slots and gate weights, all requested before any is used
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(p.slot + t * k, static_cast<int64_t>(k) * 4);
  const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(p.topk_w + t * k, static_cast<int64_t>(k) * 4);
  int sl[KM];
  float wj[KM], acc[KM];
#pragma unroll
  for (int q = 0; q < KM; ++q) {
    sl[q] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rs, q * 4u, 0, 0));
    wj[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, q * 4u, 0, 0));
  }
#pragma unroll
  for (int q = 0; q < KM; ++q) {
    sl[q] = q < k ? checked_slot(sl[q], p.rows, p.dbg, kDbgBwdSlot) : -1;
    acc[q] = 0.0f;
  }
  // dy and the kept slots' y_perm rows of up to kP columns of 4 per thread are
  // all requested before any dE store: a load issued after a store would wait
  // for that store too. A dropped slot's offsets are out of range (its rows
  // read zeros, its stores are dropped).
  constexpr int kP = KM <= 4 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rdy = uniform_rsrc(p.dy + t * H, static_cast<int64_t>(H) * 4);
  const __amdgpu_buffer_rsrc_t ry = uniform_rsrc(p.y_perm, p.rows * H * 4);
  const __amdgpu_buffer_rsrc_t rd = uniform_rsrc(p.dE, p.rows * H * 2);
  const int nc = H / 4;
  for (int c0 = threadIdx.x; c0 < nc; c0 += kP * 256) {
    f32x4_t d[kP], e[kP][KM];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int c = c0 + i * 256;
      const bool cv = c < nc;
      d[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rdy, cv ? c * 16u : kOOB, 0, kReadOnce));
#pragma unroll
      for (int q = 0; q < KM; ++q) {
        const uint32_t off = (cv && sl[q] >= 0) ? (static_cast<uint32_t>(sl[q]) * H + c * 4) * 4u : kOOB;
        e[i][q] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, kReadOnce));
      }
    }
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      const int c = c0 + i * 256;
      const bool cv = c < nc;
#pragma unroll
      for (int q = 0; q < KM; ++q) {
        acc[q] = fmaf(d[i][0], e[i][q][0], fmaf(d[i][1], e[i][q][1], fmaf(d[i][2], e[i][q][2], fmaf(d[i][3], e[i][q][3], acc[q]))));
        const float sw = s * wj[q];
        const uint32_t lo = f32_to_bf16(sw * d[i][0]) | (static_cast<uint32_t>(f32_to_bf16(sw * d[i][1])) << 16);
        const uint32_t hi = f32_to_bf16(sw * d[i][2]) | (static_cast<uint32_t>(f32_to_bf16(sw * d[i][3])) << 16);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const uint32_t off = (cv && sl[q] >= 0) ? (static_cast<uint32_t>(sl[q]) * H + c * 4) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, rd, off, 0, 0);
      }
    }
  }
  // dw_j = s <dy, E_j>: each wave's sums, then the four waves in order
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < KM; ++q) {
    const float v = wave_sum(acc[q]);
    if ((threadIdx.x & 63) == 0) red[wave][q] = v;
  }
  __syncthreads();
  if (threadIdx.x < KM) {
    const int q = threadIdx.x;
    const float v = ((red[0][q] + red[1][q]) + red[2][q]) + red[3][q];
    int sq = -1;
#pragma unroll
    for (int u = 0; u < KM; ++u)
      if (u == q) sq = sl[u];
    if (q < k) s_dw[q] = sq >= 0 ? s * v : 0.0f;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  gate_to_logits(p, t, s_dw);
}

// dx[t] = sum over kept slots of dx_perm[slot] (in slot order) + the router
// terms sum_n dlog[t,n] W_g[:,n] (+ dnz[t,n] W_noise[:,n]). A block owns
// kTokB tokens, so each router weight row is read once per kTokB tokens; a
// thread owns 4 consecutive h and reads their W_g rows as 16-byte vectors.
constexpr int kTokB = 4;
__global__ __launch_bounds__(256) void k_bwd_dx(BwdDxParams p) {
  __shared__ float s_dl[kTokB][64], s_dn[kTokB][64];
  __shared__ int s_sl[kTokB][8];
  static_assert(kTokB * 8 <= 256 && kTokB * 64 <= 1024, "one pass of the staging loops");
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokB;
  const int H = p.H, N = p.N, k = p.k;
  for (int i = threadIdx.x; i < kTokB * 64; i += 256) {
    const int tt = i / 64, n = i % 64;
    const bool ok = t0 + tt < p.T && n < N;
    s_dl[tt][n] = ok ? p.dlog[(t0 + tt) * N + n] : 0.0f;
    s_dn[tt][n] = (ok && p.noisy) ? p.dnz[(t0 + tt) * N + n] : 0.0f;
  }
  for (int i = threadIdx.x; i < kTokB * 8; i += 256) {
    const int tt = i / 8, j = i % 8;
    s_sl[tt][j] = (t0 + tt < p.T && j < k) ? checked_slot(p.slot[(t0 + tt) * k + j], p.rows, p.dbg, kDbgBwdSlot) : -1;
  }
  __syncthreads();
  const bool vec = (N % 4) == 0;
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    f32x4_t acc[kTokB];
#pragma unroll
    for (int tt = 0; tt < kTokB; ++tt) {
      acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (t0 + tt >= p.T) continue;
      if (k <= 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int sl = s_sl[tt][j];
          if (sl >= 0) acc[tt] += *reinterpret_cast<const f32x4_t*>(p.dx_perm + static_cast<int64_t>(sl) * H + c * 4);
        }
      } else {
        for (int j = 0; j < k; ++j) {
          const int sl = checked_slot(p.slot[(t0 + tt) * k + j], p.rows, p.dbg, kDbgBwdSlot);
          if (sl >= 0) acc[tt] += *reinterpret_cast<const f32x4_t*>(p.dx_perm + static_cast<int64_t>(sl) * H + c * 4);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t h = c * 4 + q;
      for (int n0 = 0; n0 < N; n0 += 4) {
        f32x4_t wg = {0.0f, 0.0f, 0.0f, 0.0f}, wn = {0.0f, 0.0f, 0.0f, 0.0f};
        if (vec) {
          wg = *reinterpret_cast<const f32x4_t*>(p.Wg + h * N + n0);
          if (p.noisy) wn = *reinterpret_cast<const f32x4_t*>(p.Wn + h * N + n0);
        } else {
          for (int e = 0; e < 4 && n0 + e < N; ++e) {
            wg[e] = p.Wg[h * N + n0 + e];
            if (p.noisy) wn[e] = p.Wn[h * N + n0 + e];
          }
        }
#pragma unroll
        for (int tt = 0; tt < kTokB; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[tt][q] = fmaf(s_dl[tt][n0 + e], wg[e], fmaf(s_dn[tt][n0 + e], wn[e], acc[tt][q]));
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTokB; ++tt)
      if (t0 + tt < p.T) *reinterpret_cast<f32x4_t*>(p.dx + (t0 + tt) * H + c * 4) = acc[tt];
  }
}

// The same sums for N (times two when noisy) of at most 32 router columns and
// at most KM slots, with the router weights read once per kTokX tokens: a
// block owns kTokX tokens and 1024 columns of H (256 threads, 4 consecutive h
// each), and each thread keeps its 4 rows of W_g (and W_noise) in registers.
// The slot rows of kU tokens are requested together as buffer loads (a
// dropped slot's offset is out of range and reads zeros), a batch ahead.
// Per element the order is that of k_bwd_dx: the slots in order, then the
// router terms in expert order (the clean gate skips the noise terms, which
// add zeros there).
constexpr int kTokX = 32;
template <int NM, bool NOISY, int KM>
__global__ __launch_bounds__(256) void k_bwd_dx_regs(BwdDxParams p) {
  constexpr int kU = KM <= 2 ? 4 : 2;
  __shared__ float s_dl[kTokX][NM], s_dn[NOISY ? kTokX : 1][NM];
  __shared__ int s_sl[kTokX][KM];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokX;
  const int H = p.H, N = p.N, k = p.k;
  for (int i = threadIdx.x; i < kTokX * NM; i += 256) {
    const int tt = i / NM, n = i % NM;
    const bool ok = t0 + tt < p.T && n < N;
    s_dl[tt][n] = ok ? p.dlog[(t0 + tt) * N + n] : 0.0f;
    if (NOISY) s_dn[tt][n] = ok ? p.dnz[(t0 + tt) * N + n] : 0.0f;
  }
  for (int i = threadIdx.x; i < kTokX * KM; i += 256) {
    const int tt = i / KM, j = i % KM;
    s_sl[tt][j] = (t0 + tt < p.T && j < k) ? checked_slot(p.slot[(t0 + tt) * k + j], p.rows, p.dbg, kDbgBwdSlot) : -1;
  }
  const int h0 = (blockIdx.y * 256 + threadIdx.x) * 4;
  const bool hv = h0 < H;  // H % 4 == 0
  // the thread's 4 rows of W are 4 N contiguous floats: 16-byte loads when
  // N % 4 == 0 (columns past N read as zero through the range check)
  float wg[4][NM], wn[NOISY ? 4 : 1][NM];
  if (N % 4 == 0) {
    const __amdgpu_buffer_rsrc_t rg = uniform_rsrc(p.Wg, static_cast<int64_t>(H) * N * 4);
    const __amdgpu_buffer_rsrc_t rn = uniform_rsrc(NOISY ? p.Wn : p.Wg, static_cast<int64_t>(H) * N * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NM; n += 4) {
        const uint32_t off = (hv && n < N) ? static_cast<uint32_t>((h0 + q) * N + n) * 4u : kOOB;
        const f32x4_t a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) wg[q][n + e] = a[e];
        if (NOISY) {
          const f32x4_t b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rn, off, 0, 0));
#pragma unroll
          for (int e = 0; e < 4; ++e) wn[q][n + e] = b[e];
        }
      }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NM; ++n) {
        const bool ok = hv && n < N;
        wg[q][n] = ok ? p.Wg[static_cast<int64_t>(h0 + q) * N + n] : 0.0f;
        if (NOISY) wn[q][n] = ok ? p.Wn[static_cast<int64_t>(h0 + q) * N + n] : 0.0f;
      }
  }
  const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(p.dx_perm, p.rows * H * 4);
  __syncthreads();
  if (!hv) return;
  const int tend = static_cast<int>(min(static_cast<int64_t>(kTokX), p.T - t0));
  // double-buffered: the slot rows of the next kU tokens are requested before
  // this batch is summed and stored
  f32x4_t v[2][kU][KM];
  auto load = [&](f32x4_t (&dst)[kU][KM], int tb) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const int sl = tb + u < tend ? s_sl[tb + u][j] : -1;
        const uint32_t off = sl >= 0 ? (static_cast<uint32_t>(sl) * static_cast<uint32_t>(H) + h0) * 4u : kOOB;
        dst[u][j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kReadOnce));
      }
  };
  auto finish = [&](const f32x4_t (&src)[kU][KM], int tb) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (tb + u >= tend) break;
      const int tt = tb + u;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < KM; ++j) acc += src[u][j];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int n = 0; n < NM; ++n)
          acc[q] = NOISY ? fmaf(s_dl[tt][n], wg[q][n], fmaf(s_dn[tt][n], wn[q][n], acc[q]))
                         : fmaf(s_dl[tt][n], wg[q][n], acc[q]);
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4_t*>(p.dx + (t0 + tt) * H + h0));
    }
  };
  load(v[0], 0);
  for (int tb = 0; tb < tend; tb += 2 * kU) {
    load(v[1], tb + kU);
    finish(v[0], tb);
    if (tb + 2 * kU < tend) load(v[0], tb + 2 * kU);
    finish(v[1], tb + kU);
  }
}

// Router weight gradients dW_g = x^T dlog and dW_noise = x^T dnz, in two
// passes for a fixed summation order: pass 1 sums a chunk of kTokW tokens per
// block into partials [chunk][N (+N)][H] (thread = HPT consecutive h with one
// vector load of x per token, all N), pass 2 adds the chunks in order.
constexpr int kTokW = 32;
constexpr int kRwThreads = 128;

// v[0..HPT)[n] to dst[0..HPT) with 16-byte (or narrower) vector stores
template <int HPT, int NM>
__device__ __forceinline__ void store_run(float* dst, const float (&v)[HPT][NM], int n) {
  if constexpr (HPT >= 4) {
#pragma unroll
    for (int q = 0; q < HPT; q += 4)
      *reinterpret_cast<f32x4_t*>(dst + q) = f32x4_t{v[q][n], v[q + 1][n], v[q + 2][n], v[q + 3][n]};
  } else if constexpr (HPT == 2) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f32x2_t*>(dst) = f32x2_t{v[0][n], v[1][n]};
  } else {
    dst[0] = v[0][n];
  }
}
template <int NMAX, bool NOISY, int HPT>
__global__ __launch_bounds__(kRwThreads) void k_router_wgrad(RouterWgradParams p) {
  __shared__ float s_dl[kTokW][NMAX], s_dn[NOISY ? kTokW : 1][NMAX];
  const int h0 = (blockIdx.x * kRwThreads + threadIdx.x) * HPT;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTokW;
  const int N = p.N;
  for (int i = threadIdx.x; i < kTokW * NMAX; i += kRwThreads) {
    const int tt = i / NMAX, n = i % NMAX;
    const bool ok = t0 + tt < p.T && n < N;
    s_dl[tt][n] = ok ? p.dlog[(t0 + tt) * N + n] : 0.0f;
    if (NOISY) s_dn[tt][n] = ok ? p.dnz[(t0 + tt) * N + n] : 0.0f;
  }
  __syncthreads();
  if (h0 >= p.H) return;
  float a[HPT][NMAX], b[HPT][NOISY ? NMAX : 1];
#pragma unroll
  for (int q = 0; q < HPT; ++q)
#pragma unroll
    for (int n = 0; n < NMAX; ++n) {
      a[q][n] = 0.0f;
      if (NOISY) b[q][n] = 0.0f;
    }
  const int tn = static_cast<int>(min(static_cast<int64_t>(kTokW), p.T - t0));
  // x of the next kPre tokens is requested before their products, so the
  // loads overlap instead of each waiting out a memory round trip
  constexpr int kPre = 8;
  for (int tb = 0; tb < tn; tb += kPre) {
  uint16_t xraw[kPre][HPT];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int tt = min(tb + u, tn - 1);
    const uint16_t* xr = p.x + (t0 + tt) * p.H + h0;
    if constexpr (HPT == 8) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xraw[u][2 * q] = static_cast<uint16_t>(v[q]);
        xraw[u][2 * q + 1] = static_cast<uint16_t>(v[q] >> 16);
      }
    } else if constexpr (HPT == 4) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(xr);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        xraw[u][2 * q] = static_cast<uint16_t>(v[q]);
        xraw[u][2 * q + 1] = static_cast<uint16_t>(v[q] >> 16);
      }
    } else if constexpr (HPT == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(xr);
      xraw[u][0] = static_cast<uint16_t>(v);
      xraw[u][1] = static_cast<uint16_t>(v >> 16);
    } else {
      xraw[u][0] = xr[0];
    }
  }
  // every value is converted before any use that depends on the token count,
  // so the compiler keeps the kPre loads issued together
  float xv[kPre][HPT];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
#pragma unroll
    for (int q = 0; q < HPT; ++q) xv[u][q] = bf16_to_f32(xraw[u][q]);
  const int cnt = min(kPre, tn - tb);
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int tt = tb + u;
    // a token past the chunk's end adds 0 (its slot of the staged gradients is 0)
    const float live = u < cnt ? 1.0f : 0.0f;
    const int ts = u < cnt ? tt : 0;
#pragma unroll
    for (int q = 0; q < HPT; ++q)
#pragma unroll
      for (int n = 0; n < NMAX; ++n) {
        a[q][n] = fmaf(xv[u][q] * live, s_dl[ts][n], a[q][n]);
        if (NOISY) b[q][n] = fmaf(xv[u][q] * live, s_dn[ts][n], b[q][n]);
      }
  }
  }
  // partials [chunk][column][H]: a lane stores its HPT consecutive h of one
  // column as one vector, so a wave's store covers contiguous memory
  const int per = N * (NOISY ? 2 : 1);
  float* out = p.part + static_cast<int64_t>(blockIdx.y) * per * p.H + h0;
#pragma unroll
  for (int n = 0; n < NMAX; ++n)
    if (n < N) {
      store_run<HPT>(out + static_cast<int64_t>(n) * p.H, a, n);
      if (NOISY) store_run<HPT>(out + static_cast<int64_t>(N + n) * p.H, b, n);
    }
}

// Pass 2: each output's chunks in order. Four threads share an output, each
// adding a contiguous quarter of the chunks (sixteen loads in flight), and
// the quarters are added in order.
constexpr int kSumQ = 4;
__global__ __launch_bounds__(64 * kSumQ) void k_router_wgrad_sum(RouterWgradParams p, int chunks) {
  __shared__ float s_q[kSumQ][64];
  const int per = p.N * (p.noisy ? 2 : 1);
  const int64_t total = static_cast<int64_t>(p.H) * per;
  const int q = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + o;  // column * H + h
  const int cq = (chunks + kSumQ - 1) / kSumQ;
  const int c0 = q * cq, c1 = min(chunks, c0 + cq);
  float v = 0.0f;
  if (i < total) {
    for (int cb = c0; cb < c1; cb += 16) {
      float u[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) u[j] = cb + j < c1 ? p.part[static_cast<int64_t>(cb + j) * total + i] : 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) v += u[j];
    }
  }
  s_q[q][o] = v;
  __syncthreads();
  if (q != 0 || i >= total) return;
  float r = s_q[0][o];
#pragma unroll
  for (int w = 1; w < kSumQ; ++w) r += s_q[w][o];
  const int64_t n = i / p.H, h = i % p.H;
  if (n < p.N) p.dWg[h * p.N + n] = r;
  else p.dWn[h * p.N + (n - p.N)] = r;
}

// Any k (up to 64): slots in groups of eight, loads as they come.
__global__ __launch_bounds__(256) void k_bwd_gate_any(BwdGateParams p) {
  __shared__ float red[4];
  __shared__ float s_dw[64];
  const int64_t t = blockIdx.x;
  if (t == 0 && p.zero)
    for (int i = threadIdx.x; i < p.zero_n; i += 256) p.zero[i] = 0;
  const int H = p.H, k = p.k, N = p.N;
  const float s = p.scale;
  const float* dy = p.dy + t * H;
  for (int j0 = 0; j0 < k; j0 += 8) {
    int sl[8];
    float wj[8], acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q;
      sl[q] = j < k ? checked_slot(p.slot[t * k + j], p.rows, p.dbg, kDbgBwdSlot) : -1;
      wj[q] = j < k ? p.topk_w[t * k + j] : 0.0f;
      acc[q] = 0.0f;
    }
    for (int c = threadIdx.x; c < H / 4; c += 256) {
      const f32x4_t d = *reinterpret_cast<const f32x4_t*>(dy + c * 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (sl[q] < 0) continue;
        const f32x4_t e = *reinterpret_cast<const f32x4_t*>(p.y_perm + static_cast<int64_t>(sl[q]) * H + c * 4);
        acc[q] = fmaf(d[0], e[0], fmaf(d[1], e[1], fmaf(d[2], e[2], fmaf(d[3], e[3], acc[q]))));
        const float sw = s * wj[q];
        const uint32_t lo = f32_to_bf16(sw * d[0]) | (static_cast<uint32_t>(f32_to_bf16(sw * d[1])) << 16);
        const uint32_t hi = f32_to_bf16(sw * d[2]) | (static_cast<uint32_t>(f32_to_bf16(sw * d[3])) << 16);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2_t*>(p.dE + static_cast<int64_t>(sl[q]) * H + c * 4) = u32x2_t{lo, hi};
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (j0 + q >= k) break;
      const float v = block_sum(acc[q], red);  // same value on every thread
      if (threadIdx.x == 0) s_dw[j0 + q] = sl[q] >= 0 ? s * v : 0.0f;
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  gate_to_logits(p, t, s_dw);
}

}  // namespace

hipError_t launch_bwd_gate(const BwdGateParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.T)), block(256);
  if (p.k <= 2) hipLaunchKernelGGL(k_bwd_gate<2>, grid, block, 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL(k_bwd_gate<4>, grid, block, 0, s, p);
  else if (p.k <= 8) hipLaunchKernelGGL(k_bwd_gate<8>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(k_bwd_gate_any, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (p.k <= 4 && p.N <= (p.noisy ? 16 : 32)) {
    const dim3 grid(static_cast<unsigned>((p.T + kTokX - 1) / kTokX), static_cast<unsigned>((p.H / 4 + 255) / 256));
#define MOE_DX(NM, NZ)                                                                         \
  do {                                                                                         \
    if (p.k <= 2) hipLaunchKernelGGL((k_bwd_dx_regs<NM, NZ, 2>), grid, dim3(256), 0, s, p);    \
    else hipLaunchKernelGGL((k_bwd_dx_regs<NM, NZ, 4>), grid, dim3(256), 0, s, p);             \
  } while (0)
    if (p.noisy) {
      if (p.N <= 8) MOE_DX(8, true); else MOE_DX(16, true);
    } else {
      if (p.N <= 8) MOE_DX(8, false); else if (p.N <= 16) MOE_DX(16, false); else MOE_DX(32, false);
    }
#undef MOE_DX
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_bwd_dx, dim3(static_cast<unsigned>((p.T + kTokB - 1) / kTokB)), dim3(256), 0, s, p);
  return hipGetLastError();
}

int router_wgrad_chunks(int64_t T) { return static_cast<int>((T + kTokW - 1) / kTokW); }

hipError_t launch_router_wgrad(const RouterWgradParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  // h per thread: as many as keep the accumulators within 128 registers
  // (H % 8 == 0, so every width divides H)
  const int per = (p.N <= 8 ? 8 : p.N <= 16 ? 16 : p.N <= 32 ? 32 : 64) * (p.noisy ? 2 : 1);
  const int hpt = per <= 16 ? 8 : per <= 32 ? 4 : per <= 64 ? 2 : 1;
  const dim3 grid((p.H / hpt + kRwThreads - 1) / kRwThreads, router_wgrad_chunks(p.T));
#define MOE_RW(NM, NZ, HP) hipLaunchKernelGGL((k_router_wgrad<NM, NZ, HP>), grid, dim3(kRwThreads), 0, s, p)
  if (p.N <= 8) {
    if (p.noisy) MOE_RW(8, true, 8); else MOE_RW(8, false, 8);
  } else if (p.N <= 16) {
    if (p.noisy) MOE_RW(16, true, 4); else MOE_RW(16, false, 8);
  } else if (p.N <= 32) {
    if (p.noisy) MOE_RW(32, true, 2); else MOE_RW(32, false, 4);
  } else {
    if (p.noisy) MOE_RW(64, true, 1); else MOE_RW(64, false, 2);
  }
#undef MOE_RW
  (void)hpt;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(p.H) * p.N * (p.noisy ? 2 : 1);
  hipLaunchKernelGGL(k_router_wgrad_sum, dim3(static_cast<unsigned>((n + 63) / 64)), dim3(64 * kSumQ), 0, s, p,
                     router_wgrad_chunks(p.T));
  return hipGetLastError();
}

}  // namespace moe
