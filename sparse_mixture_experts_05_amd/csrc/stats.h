// Fixed-order reduction of the router's per-block statistics, shared by the
// standalone statistics kernel and the persistent expert kernel (which runs it
// in one workgroup once its queue is empty), so both give the same bits.
//
// Load, importance and P follow the LLaMA-MoE v2 article's gating section
// (balance loss) and the LLaMA-MoE monitoring list: load_i = assignments to
// expert i before capacity, importance_i = sum of its gate weights,
// P_i = mean over tokens of softmax(logits)_i, balance = sum_i f_i P_i with
// f_i = load_i / (T k). The smooth load is the sum over tokens of the
// router's per-token probabilities (see the routers).
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStatGroups = 8;  // waves of the reducing workgroup, one group of router blocks each
// LDS the reduction needs (8-byte aligned)
constexpr int kStatLdsBytes = kStatGroups * 64 * (8 + 4 + 4 + 4) + 64 * 4;

// Run by every thread of a workgroup of at least kStatGroups * 64 threads
// (threads past that take no part). Group g (one wave) sums a contiguous range
// of router blocks in block order, lane n holding expert n; wave 0 then adds
// the group partials in group order. The order depends only on the block
// count, so the result is the same on every run.
__device__ inline void stats_reduce(const StatsParams& p, void* lds) {
  int64_t* s_cnt = static_cast<int64_t*>(lds);                 // [kStatGroups][64]
  float* s_imp = reinterpret_cast<float*>(s_cnt + kStatGroups * 64);  // [kStatGroups][64]
  float* s_ps = s_imp + kStatGroups * 64;                         // [kStatGroups][64]
  float* s_sl = s_ps + kStatGroups * 64;                          // [kStatGroups][64]
  float* s_fp = s_sl + kStatGroups * 64;                          // [64]
  constexpr int S = kStatsPerExpert;
  const int n = threadIdx.x & 63, g = threadIdx.x >> 6;
  const bool part = g < kStatGroups;
  const bool valid = part && n < p.N;
  const int b0 = static_cast<int>(static_cast<int64_t>(p.blocks) * g / kStatGroups);
  const int b1 = static_cast<int>(static_cast<int64_t>(p.blocks) * (g + 1) / kStatGroups);
  int64_t c = 0;
  float imp = 0.0f, ps = 0.0f, sl = 0.0f;
  if (valid) {
    constexpr int U = 8;  // loads issued together before the in-order adds
    for (int b = b0; b < b1; b += U) {
      int hv[U];
      float iv[U], pv[U], sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bb = b + u < b1 ? b + u : b;
        const float* part = p.stat_part + (static_cast<int64_t>(bb) * p.N + n) * S;
        hv[u] = p.hist[static_cast<int64_t>(bb) * p.N + n];
        iv[u] = part[0];
        pv[u] = part[1];
        sv[u] = part[2];
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (b + u < b1) {
          c += hv[u];
          imp += iv[u];
          ps += pv[u];
          sl += sv[u];
        }
    }
  }
  if (part) {
    s_cnt[g * 64 + n] = c;
    s_imp[g * 64 + n] = imp;
    s_ps[g * 64 + n] = ps;
    s_sl[g * 64 + n] = sl;
  }
  __syncthreads();
  if (g != 0) return;
  c = 0;
  imp = 0.0f;
  ps = 0.0f;
  sl = 0.0f;
#pragma unroll
  for (int q = 0; q < kStatGroups; ++q) {
    c += s_cnt[q * 64 + n];
    imp += s_imp[q * 64 + n];
    ps += s_ps[q * 64 + n];
    sl += s_sl[q * 64 + n];
  }
  const bool vn = n < p.N;
  const float load = static_cast<float>(c);
  if (vn && p.load) p.load[n] = static_cast<int32_t>(c);
  const float Pn = p.T > 0 ? ps / static_cast<float>(p.T) : 0.0f;
  const float fn = p.T > 0 ? load / (static_cast<float>(p.T) * static_cast<float>(p.k)) : 0.0f;
  // balance = sum_i f_i P_i, summed in expert order by lane 0
  s_fp[n] = vn ? fn * Pn : 0.0f;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (vn) {
    if (p.importance) p.importance[n] = imp;
    if (p.P) p.P[n] = Pn;
    if (p.smooth_load) p.smooth_load[n] = sl;
  }
  if (n == 0 && p.balance) {
    float b = 0.0f;
    for (int i = 0; i < p.N; ++i) b += s_fp[i];
    p.balance[0] = b;
  }
}

}  // namespace moe
