// Capacity clip and permutation of (token, expert) assignments into
// expert-contiguous order, without atomics.
//
// Each expert keeps its assignments in token order up to its capacity; the
// rest overflow and are dropped ("Llama 3 Meets MoE" review, section 3,
// capacity factor). The rank of an assignment inside its expert's queue is
//   (assignments to that expert in earlier router blocks, from the per-block
//    histogram) + (earlier waves of this block) + (earlier lanes of this wave)
// where the last two come from wave ballots and popcounts. Ranks are unique
// and exact, so the whole permutation is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kScatterThreads = 256;

// Histogram of topk_idx with the router's block granularity (one block of
// 64 threads per router block; thread n counts expert n).
__global__ __launch_bounds__(64) void k_hist(HistParams p) {
  const int n = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * p.tokens_per_block;
  int64_t t1 = t0 + p.tokens_per_block;
  if (t1 > p.T) t1 = p.T;
  int c = 0;
  for (int64_t t = t0; t < t1; ++t)
    for (int j = 0; j < p.k; ++j) c += (p.topk_idx[t * p.k + j] == n) ? 1 : 0;
  if (n < p.N) p.hist[static_cast<int64_t>(blockIdx.x) * p.N + n] = c;
}

template <int KMAX>
__global__ __launch_bounds__(kScatterThreads) void k_scatter(ScatterParams p) {
  __shared__ int s_base[64], s_tot[64], s_kept[64], s_off[65];
  __shared__ int s_wcnt[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, k = p.k;
  const int64_t T = p.T;
  const int64_t tb0 = static_cast<int64_t>(blockIdx.x) * kScatterThreads;
  const int64_t nhb = (T + p.hist_tokens - 1) / p.hist_tokens;
  const int64_t hb0 = tb0 / p.hist_tokens;

  // this thread's token; its expert list is loaded first so that the load
  // overlaps the histogram reads below
  const int64_t t = tb0 + tid;
  const bool tv = t < T;
  int idx[KMAX], pre[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    idx[j] = (tv && j < k) ? p.topk_idx[t * k + j] : -1;
    pre[j] = 0;
  }

  // per-expert totals and the count before this block: every thread reads
  // its share of the histogram at once and adds it into LDS (integer sums,
  // so the order of the adds does not matter)
  if (tid < 64) {
    s_base[tid] = 0;
    s_tot[tid] = 0;
  }
  __syncthreads();
  {
    const int64_t nel = nhb * N;
    const int64_t split = hb0 * N;  // elements before this block's first histogram row
    constexpr int U = 16;  // loads in flight per thread before their adds (4096 counts in one round trip)
    if (kScatterThreads % N == 0) {
      // every element this thread reads is a count of expert tid % N: sum in
      // registers, then one LDS add per counter instead of one per element
      int tot = 0, base = 0;
      for (int64_t i0 = tid; i0 < nel; i0 += U * kScatterThreads) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = i0 + u * kScatterThreads;
          v[u] = i < nel ? p.hist[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tot += v[u];
          if (i0 + u * kScatterThreads < split) base += v[u];
        }
      }
      if (tot) atomicAdd(&s_tot[tid % N], tot);
      if (base) atomicAdd(&s_base[tid % N], base);
    } else {
      for (int64_t i0 = tid; i0 < nel; i0 += U * kScatterThreads) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = i0 + u * kScatterThreads;
          v[u] = i < nel ? p.hist[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = i0 + u * kScatterThreads;
          const int n = static_cast<int>(i % N);
          if (v[u]) {
            atomicAdd(&s_tot[n], v[u]);
            if (i < split) atomicAdd(&s_base[n], v[u]);
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid < N) {
    const int c = s_tot[tid];
    s_kept[tid] = p.capacity < 0 ? c : (c < p.capacity ? c : p.capacity);
    if (blockIdx.x == 0) {
      if (p.counts) p.counts[tid] = c;
      if (p.kept) p.kept[tid] = s_kept[tid];
    }
  }
  __syncthreads();
  if (tid == 0) {
    s_off[0] = 0;
    for (int e = 0; e < N; ++e) s_off[e + 1] = s_off[e] + s_kept[e];
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid <= N) p.offsets[tid] = s_off[tid];
  if (blockIdx.x == 0 && p.zero)
    for (int i = tid; i < p.zero_n; i += kScatterThreads) p.zero[i] = 0;

  // rank among the wave's earlier assignments, per expert, by ballot: every
  // slot of earlier lanes, then the earlier slots of the same token (a row of
  // topk_idx from a caller may name one expert twice; each entry is its own
  // assignment, in (token, slot) order)
  for (int e = 0; e < N; ++e) {
    int before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {  // uniform over the wave
        const uint64_t m = __ballot(idx[j] == e);
        total += __popcll(m);
        before += __popcll(m & lanemask_lt());
      }
    }
    if (lane == 0) s_wcnt[wave][e] = total;
    int same = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (idx[j] == e) pre[j] = before + same++;
  }
  __syncthreads();
  if (tv) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        // an expert index outside [0, N) (possible only in a caller's
        // topk_idx) is dropped; the row bound guards against a histogram
        // that disagrees with topk_idx
        const int e = idx[j];
        const bool ve = e >= 0 && e < N;
        int rank = 0;
        if (ve) {
          int woff = 0;
          for (int w = 0; w < wave; ++w) woff += s_wcnt[w][e];
          rank = s_base[e] + woff + pre[j];
        }
        const int64_t row = ve ? static_cast<int64_t>(s_off[e]) + rank : -1;
        const bool fits = ve && (p.capacity < 0 || rank < p.capacity);
        if (fits && row >= T * k) debug_flag(p.dbg, kDbgScatterRow);
        const bool keep = fits && row < T * k;
        p.slot[t * k + j] = keep ? static_cast<int32_t>(row) : -1;
        if (keep) p.row_token[row] = static_cast<int32_t>(t);
      }
    }
  }
  // rows past the last kept one
  const int64_t A = min(static_cast<int64_t>(s_off[N]), T * k);
  for (int64_t r = A + tb0 + tid; r < T * k; r += static_cast<int64_t>(gridDim.x) * kScatterThreads)
    p.row_token[r] = -1;
}

// x_perm[r] = x[row_token[r]] for r < offsets[N]; one wave per row.
__global__ __launch_bounds__(256) void k_gather(GatherParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t A = min(static_cast<int64_t>(p.offsets[p.N]), p.rows_max);
  if (r >= A) return;
  const int64_t src = p.row_token[r];
  const int64_t row_bytes = static_cast<int64_t>(p.H) * p.elem_bytes;
  char* d = static_cast<char*>(p.x_perm) + r * row_bytes;
  if (src < 0 || src >= p.T) {  // never from the scatter; a guard against a row index outside x
    debug_flag(p.dbg, kDbgGatherRow);
    for (int64_t o = lane * 16; o < row_bytes; o += 64 * 16) *reinterpret_cast<u32x4_t*>(d + o) = u32x4_t{0, 0, 0, 0};
    return;
  }
  const char* s = static_cast<const char*>(p.x) + src * row_bytes;
  // eight 16-byte pieces per lane are loaded before they are stored: a load
  // issued after a store would also wait for that store
  for (int64_t o0 = lane * 16; o0 < row_bytes; o0 += 8 * 64 * 16) {
    u32x4_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t o = o0 + i * 64 * 16;
      v[i] = o < row_bytes ? *reinterpret_cast<const u32x4_t*>(s + o) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t o = o0 + i * 64 * 16;
      if (o < row_bytes) *reinterpret_cast<u32x4_t*>(d + o) = v[i];
    }
  }
}

}  // namespace

hipError_t launch_hist(const HistParams& p, hipStream_t s) {
  const int64_t blocks = (p.T + p.tokens_per_block - 1) / p.tokens_per_block;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_hist, dim3(static_cast<unsigned>(blocks)), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
  const int64_t blocks = (p.T + kScatterThreads - 1) / kScatterThreads;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kScatterThreads);
  if (p.k <= 2) hipLaunchKernelGGL(k_scatter<2>, grid, block, 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL(k_scatter<4>, grid, block, 0, s, p);
  else if (p.k <= 8) hipLaunchKernelGGL(k_scatter<8>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(k_scatter<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  const int64_t blocks = (p.rows_max + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
