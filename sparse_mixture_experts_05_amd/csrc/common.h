// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element access for the two activation / weight storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Butterfly sum over the 64 lanes. Every lane ends with the bitwise-same
// value: at each level lanes i and i^m add the same two numbers, and fp32
// addition is commutative.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float softplus(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

constexpr uint32_t kOOB = 0xFFFFFFF0u;    // byte offset past any buffer: loads return zero
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data

// A wave-uniform buffer descriptor: the base address passes through
// readfirstlane so the descriptor lives in scalar registers (a descriptor in
// vector registers makes every load a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  const int num = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < 0x7FFFFFF0 ? bytes : 0x7FFFFFF0));
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, num, kBufferFlags);
}

// Expert e's segment of the permuted rows, [off, off + cnt), from the
// device-side offsets, clamped to [0, rows_max): offsets that a caller
// passes in (or that disagree with the row bound the workspace was sized
// for) can then never move a tile's loads or stores past its buffers.
// Bounds invariants. Every index that data can steer is guarded in every
// build (the access is skipped or clamped); a debug build (-DMOE_DEBUG) also
// records a guard that fires by raising `bit` of the workspace's debug word
// (dbg may be null: nothing recorded). On valid data no guard fires.
constexpr int kDbgScatterRow = 1;   // a kept slot's row at or past T*k
constexpr int kDbgGatherRow = 2;    // a row_token entry outside x's rows
constexpr int kDbgCombineSlot = 4;  // a slot at or past y_perm's rows
constexpr int kDbgOffsets = 8;      // offsets outside [0, rows_max] or decreasing
constexpr int kDbgBwdSlot = 16;     // the backward: a slot at or past the rows
__device__ __forceinline__ void debug_flag(int32_t* dbg, int bit) {
#ifdef MOE_DEBUG
  if (dbg) __hip_atomic_fetch_or(dbg, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  (void)dbg;
  (void)bit;
#endif
}

// A slot of a buffer of `rows` rows: the slot itself when it is in range,
// else -1 (a dropped slot), raising `bit`.
__device__ __forceinline__ int checked_slot(int s, int64_t rows, int32_t* dbg, int bit) {
  if (s >= rows) {
    debug_flag(dbg, bit);
    return -1;
  }
  return s;
}

__device__ __forceinline__ void expert_segment(const int32_t* __restrict__ offsets, int e, int rows_max, int& off,
                                               int& cnt, int32_t* dbg = nullptr) {
  const int o0 = offsets[e], o1 = offsets[e + 1];
  const int a = min(max(o0, 0), rows_max);
  const int b = min(max(o1, a), rows_max);
  if (a != o0 || b != o1) debug_flag(dbg, kDbgOffsets);
  off = a;
  cnt = b - a;
}

// Lane e < N of a wave: expert e's segment [off, off + cnt), with the offsets
// clamped to [0, rows_max] and made non-decreasing (a running maximum over
// the experts before it), so that the segments never overlap and together
// hold at most rows_max rows whatever a caller passes; lanes >= N get empty
// segments. Valid offsets come back unchanged; any other raises kDbgOffsets.
// Every lane of the wave must call it.
__device__ __forceinline__ void expert_segment_wave(const int32_t* __restrict__ offsets, int N, int rows_max,
                                                    int& off, int& cnt, int32_t* dbg = nullptr) {
  const int lane = threadIdx.x & 63;
  const bool v = lane < N;
  const int o0 = v ? offsets[lane] : 0, o1 = v ? offsets[lane + 1] : 0;
  const int a = min(max(o0, 0), rows_max);
  int A = v ? a : 0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(A, d, 64);
    if (lane >= d) A = max(A, u);
  }
  const int B = max(A, min(max(o1, 0), rows_max));
  if (v && (A != o0 || B != o1)) debug_flag(dbg, kDbgOffsets);
  off = v ? A : 0;
  cnt = v ? B - A : 0;
}

struct TileInfo {
  int expert;
  int row0;   // first permuted row of the tile
  int rows;   // valid rows in the tile (<= BM)
};

// Map a linear m-tile index to (expert, first row, valid rows). Lane e reads
// expert e's row count; a lane-wise inclusive scan of the per-expert tile
// counts locates the expert. Returns false past the last tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int N, int rows_max, int mt,
                                          TileInfo& ti, int32_t* dbg = nullptr) {
  const int lane = threadIdx.x & 63;
  int off = 0, cnt = 0;
  expert_segment_wave(offsets, N, rows_max, off, cnt, dbg);
  const int tl = (cnt + BM - 1) / BM;
  int incl = tl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  const int total = __shfl(incl, 63, 64);
  if (mt >= total) return false;
  const int e = __popcll(__ballot(incl <= mt));
  const int start = __shfl(incl - tl, e, 64);
  const int eoff = __shfl(off, e, 64);
  const int ecnt = __shfl(cnt, e, 64);
  const int local = mt - start;
  ti.expert = e;
  ti.row0 = eoff + local * BM;
  ti.rows = min(BM, ecnt - local * BM);
  return true;
}

}  // namespace moe
