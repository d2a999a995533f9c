// Grouped bf16 GEMMs of the SwiGLU experts on gfx950 matrix cores.
//
// Rows of expert e occupy [offsets[e], offsets[e+1]) of the permuted order.
// A workgroup owns one BM x BN output tile of one expert; it finds its expert
// on the device from `offsets` (no host synchronisation), stages A and B
// tiles of BK = 64 through LDS, and issues v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.
//
//   swiglu: B rows [0, BN/2) are Wgate rows, [BN/2, BN) the matching Wup rows;
//           each wave holds gate and up accumulators of the same columns, so
//           the epilogue forms SiLU(g) * u in registers and stores h as bf16
//           (LLaMA-MoE v2 article, code example, class Expert).
//   plain : C = A . B^T in fp32 (the down projection), optionally split over K
//           into separate partial outputs that the combine step adds in a
//           fixed order.
//
// Both operands are K-contiguous ("TN"): a 16-byte LDS read gives a lane its
// 8 bf16 MFMA operand elements. An LDS row holds BK bf16 (128 bytes for
// BK = 64, 64 bytes for BK = 32) and its 16-byte chunks are XOR-swizzled by
// row (see swz), which keeps both the row-wise global->LDS writes and the
// column-wise MFMA operand reads free of bank conflicts.
//
// Loads go straight from buffer loads into LDS (no register staging), STAGES
// deep, so several K steps of loads stay in flight; rows past the expert's
// segment and K past the range read as zero through the buffer's range check,
// without branches. k_experts_fused runs both projections of every expert in
// one persistent launch of 256 x 256 tiles (see the scheduling comment above
// it), and k_gemm_decode serves experts with few rows (see the comment above
// it).
#include "common.h"
#include "stats.h"
#include "kernels.h"

#include <type_traits>

namespace moe {

namespace {


// Element offset of 16-byte chunk `chunk` of LDS row `row`. The LDS serves a
// 16-byte read (ds_read_b128) for 16 lanes at a time over 64 four-byte banks
// (256 bytes), and the MFMA operand reads have 16 consecutive lanes read 16
// consecutive rows at one logical chunk, so those 16 rows must land in 16
// different 16-byte bank slots.
//   BK = 64 (128-byte rows): slot = 8*(r & 1) + position; the position is
//     c ^ ((r >> 1) & 7), distinct over the 8 rows of each parity.
//   BK = 32 (64-byte rows):  slot = 4*(r & 3) + position; the position is
//     c ^ ((r >> 2) & 3), distinct over the 4 rows of each r & 3.
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(BK == 64 || BK == 32, "K step");
  if constexpr (BK == 64) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ swz_key<BK>(row)) << 3);
}

// Linear tile order: XCD-aware remap of blockIdx.x (workgroups are dealt to
// the 8 XCDs round-robin, so XCD x runs blocks x, x+8, ...; the remap gives each
// XCD a contiguous range of the order below, and so a compact group of tiles
// that shares operands in its own L2), then groups of GM m-tiles with the
// m-tile index varying fastest, so tiles that read the same expert's weight
// tile run together.
__device__ __forceinline__ int xcd_remap(int bid, int G) {
  const int xcd = bid & 7, base = G >> 3, rem = G & 7;
  return xcd * base + min(xcd, rem) + (bid >> 3);
}

struct TilePos {
  TileInfo ti;
  int nt, split, kb0, kb1, KT;
};

// Decode this workgroup's tile; false when it has none (uniform over the
// workgroup).
template <int BM, int NO, int BK>
__device__ __forceinline__ bool decode_tile(const GemmParams& p, TilePos& tp) {
  constexpr int GM = BM >= 256 ? 4 : 8;  // m-tiles per group
  const int lane = threadIdx.x & 63;
  const int ntiles = (p.Nout + NO - 1) / NO;
  // per-expert m-tile counts (lane e = expert e), inclusive scan over lanes
  int eoff = 0, ecnt = 0;
  expert_segment_wave(p.offsets, p.N, static_cast<int>(p.rows_max), eoff, ecnt, p.dbg);
  const int etl = (ecnt + BM - 1) / BM;
  int incl = etl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  const int mtot = __shfl(incl, 63, 64);
  const int per_split = mtot * ntiles;
  // the grid is an upper bound on the tiles: the first `real` workgroups take
  // them, remapped over those alone, so the tiles spread over all 8 XCDs
  // (remapped over the whole grid, they would crowd onto the first XCDs and
  // leave the others only workgroups without a tile)
  const int real = min(per_split * p.splits, static_cast<int>(gridDim.x));
  if (static_cast<int>(blockIdx.x) >= real) return false;
  int L = xcd_remap(blockIdx.x, real);
  tp.split = L / per_split;
  L -= tp.split * per_split;
  const int g = L / (GM * ntiles);
  const int gm = min(GM, mtot - g * GM);
  const int r_in = L - g * GM * ntiles;
  const int mt = g * GM + r_in % gm;
  tp.nt = r_in / gm;
  const int e = __popcll(__ballot(incl <= mt));
  const int local = mt - __shfl(incl - etl, e, 64);
  // the values are wave-uniform; saying so keeps them (and the buffer
  // descriptors built from them) in scalar registers
  tp.ti.expert = __builtin_amdgcn_readfirstlane(e);
  tp.ti.row0 = __builtin_amdgcn_readfirstlane(__shfl(eoff, e, 64) + local * BM);
  tp.ti.rows = __builtin_amdgcn_readfirstlane(min(BM, __shfl(ecnt, e, 64) - local * BM));
  tp.nt = __builtin_amdgcn_readfirstlane(tp.nt);
  tp.split = __builtin_amdgcn_readfirstlane(tp.split);
  // K range of this split
  const int kper = ((p.K + p.splits - 1) / p.splits + BK - 1) / BK * BK;
  tp.kb0 = tp.split * kper;
  tp.kb1 = min(p.K, tp.kb0 + kper);
  tp.KT = tp.kb1 > tp.kb0 ? (tp.kb1 - tp.kb0 + BK - 1) / BK : 0;
  return true;
}

// LDS rows read by a wave's MFMA blocks; swiglu pairs gate block j with up
// block j + NB/2 over the same output columns.
template <int WM, int WN, int MB, int NB, int BN, bool SWIGLU>
__device__ __forceinline__ void frag_rows(int wm, int wn, int lane, int (&arow)[MB], int (&brow)[NB]) {
#pragma unroll
  for (int i = 0; i < MB; ++i) arow[i] = wm * WM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (SWIGLU) {
      const int half = NB / 2;
      const int jj = j < half ? j : j - half;
      brow[j] = (j < half ? 0 : BN / 2) + wn * (WN / 2) + jj * 32 + (lane & 31);
    } else {
      brow[j] = wn * WN + j * 32 + (lane & 31);
    }
  }
}

// ---- K-outer operands (the backward) ---------------------------------------
//
// The backward's GEMMs read operands whose rows are K rows: the expert
// weights as B of the input gradients (dh = dE . Wdown_e reads Wdown_e[h][f]
// with K = h; dx = dg . Wgate_e + du . Wup_e reads Wgate_e[f][h] with K = f),
// and every operand of the weight gradients, whose K is an expert's rows
// (dWdown_e = dE^T h, dWgate_e = dg^T x, dWup_e = du^T x). Such a "KN"
// operand is staged as it lies in memory: BK rows of the tile's 256 M (or N)
// columns, 512 bytes per LDS row. The MFMA operand wants 8 consecutive K of
// one column per lane; gfx950's transposing LDS read (ds_read_b64_tr_b16)
// gives each lane of a 16-lane group 4 consecutive rows of its column, so two
// reads make one operand. Lane i of a group points at row i / 4 of the four
// rows, columns 4 (i % 4) .. 4 (i % 4) + 3 of the group's 16.
//
// Bank conflicts: the LDS serves a 64-bit read 32 lanes at a time over 64
// banks. Those 32 lanes cover 4 rows x 32 columns; rows 512 bytes apart fall
// on the same banks, so 16-byte chunk c of row k is stored at chunk
// c ^ (4 (k & 3)): the 4 rows' 4 chunks then occupy 16 distinct chunk slots of
// one 256-byte window. The row-wise direct-to-LDS writes pick their global
// chunk with the same XOR.
constexpr int kKnCols = 256;  // columns of a KN LDS row (the tile's M or N extent)

__device__ __forceinline__ int kn_off(int k, int col) {
  return k * kKnCols + ((((col >> 3) ^ ((k & 3) << 2))) << 3) + (col & 7);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Lane offset (elements, within a KN stage) of the transposing reads of the
// 32-column block at column c0, K slice ks = 0 (add ks * 16 * kKnCols for
// slice ks, 4 * kKnCols for the second read).
__device__ __forceinline__ int kn_frag_off(int c0, int lane) {
  const int k = (lane >> 5) * 8 + ((lane & 15) >> 2);
  return kn_off(k, c0 + (lane & 16) + 4 * (lane & 3));
}

__device__ __forceinline__ bf16x8_t kn_frag(const uint16_t* __restrict__ st, int off) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(st + off));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(st + off + 4 * kKnCols));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// A wave's operand fragments for the K loop, in two register sets: the LDS
// reads of one K slice are in flight while the MFMAs of the previous slice
// run. A stage's last slice lands in set 1 and its MFMAs wait for the next
// step, after the barrier, so that step's first reads overlap them instead of
// leaving the matrix cores idle. PARTIAL: only the wave's first `live` 32-row
// blocks hold rows of the expert (wave-uniform), and the rest of an expert's
// last, partly filled tile is skipped, MFMAs and operand reads alike; full
// tiles take the branch-free copy.
template <int MB, int NB, int BK, bool PARTIAL, bool AKN = false, bool BKN = false>
struct FragPipe {
  static constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "a stage's last slice must land in set 1");
  bf16x8_t af[2][MB], bfr[2][NB];

  // set 1 starts as zeros, so the carried MFMAs of the first step add exact zeros
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < MB; ++i) af[1][i] = bf16x8_t{};
#pragma unroll
    for (int j = 0; j < NB; ++j) bfr[1][j] = bf16x8_t{};
  }

  __device__ __forceinline__ void load(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                       const int (&arow)[MB], const int (&brow)[NB], int khalf, int ks, int buf,
                                       int live) {
    // TN: arow/brow are LDS rows; KN: lane offsets of the transposing reads
    const int chunk = ks * 2 + khalf;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (!PARTIAL || i < live) {
        if constexpr (AKN) af[buf][i] = kn_frag(a, arow[i] + ks * 16 * kKnCols);
        else af[buf][i] = *reinterpret_cast<const bf16x8_t*>(&a[swz<BK>(arow[i], chunk)]);
      }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if constexpr (BKN) bfr[buf][j] = kn_frag(b, brow[j] + ks * 16 * kKnCols);
      else bfr[buf][j] = *reinterpret_cast<const bf16x8_t*>(&b[swz<BK>(brow[j], chunk)]);
    }
  }

  __device__ __forceinline__ void mma(int buf, f32x16_t (&acc)[MB][NB], int live) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if (!PARTIAL || i < live)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
  }

  // one stage: slice 0's reads, then the previous stage's last slice, then
  // slices 0 .. KS-2 each behind the next slice's reads; slice KS-1 stays in set 1
  __device__ __forceinline__ void stage(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                        const int (&arow)[MB], const int (&brow)[NB], int khalf,
                                        f32x16_t (&acc)[MB][NB], int live) {
    load(a, b, arow, brow, khalf, 0, 0, live);
    __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of the MFMAs below
    mma(1, acc, live);
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      load(a, b, arow, brow, khalf, ks + 1, (ks + 1) & 1, live);
      __builtin_amdgcn_sched_barrier(0);
      mma(ks & 1, acc, live);
    }
  }
};

// Accumulator layout of a 32x32 block: lane holds column (lane & 31) and rows
// 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
//
// The stores go through a buffer descriptor that spans exactly the tile's
// valid rows, so the range check drops rows past the expert's end without a
// branch; a column past Nout gets a byte offset of at least kStoreOOB, beyond
// every descriptor (tile offsets stay far below 2^31, so the sum cannot wrap).
constexpr uint32_t kStoreOOB = 0x80000000u;
// Cache-policy bits of the epilogue stores. h is stored at device scope (sc1,
// bit 4 of the policy): such a store is coherent across the XCDs' L2s once it
// has completed, so the persistent kernel publishes a finished h tile by
// waiting for its stores instead of writing back the whole L2. y_perm (or its
// split partials) is read only by a later launch and uses the default policy.
constexpr int kHStorePolicy = 16, kYStorePolicy = 0;
// Weight gradients (the tiles with both operands K-outer) are read by no
// later launch of the step: non-temporal stores (the nt bit).
constexpr int kGradStorePolicy = 2;
// The training forward's saved g and u are read only by the backward's
// input-gradient launch, several launches later, and there only once: their
// stores and loads are non-temporal as well.
constexpr int kSaveStorePolicy = 2, kSaveLoadPolicy = 2;

// SiLU(z) = z * sigmoid(z) with the hardware exp2 and reciprocal, each within
// about one ulp of fp32, far below the bf16 rounding of h that follows.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

template <int WM, int WN, int MB, int NB, bool SWIGLU, int CPOL = kYStorePolicy>
__device__ __forceinline__ void epilogue(const GemmParams& p, const TilePos& tp, int wm, int wn, int lane, int NO,
                                         f32x16_t (&acc)[MB][NB]) {
  const int col_l = lane & 31, khalf = lane >> 5;
  const int row_l = wm * WM + khalf * 4;  // this lane's first row in the tile
  if (!SWIGLU && p.epi == 1) {
    // SwiGLU backward: the sum is dh; g and u of the same rows come from gu
    const int64_t ldg = 2 * static_cast<int64_t>(p.Nout);
    const float* gbase = p.gu + static_cast<int64_t>(tp.ti.row0) * ldg;
    const __amdgpu_buffer_rsrc_t rg = uniform_rsrc(gbase, static_cast<int64_t>(tp.ti.rows) * ldg * 4);
    const uint16_t* base = static_cast<const uint16_t*>(p.C) + static_cast<int64_t>(tp.ti.row0) * p.ldc;
    const __amdgpu_buffer_rsrc_t rc = uniform_rsrc(base, static_cast<int64_t>(tp.ti.rows) * p.ldc * 2);
    const uint32_t ld = static_cast<uint32_t>(p.ldc) * 2u, lg = static_cast<uint32_t>(ldg) * 4u;
    const uint32_t uoff_g = static_cast<uint32_t>(p.Nout) * 4u, uoff_c = static_cast<uint32_t>(p.Nout) * 2u;
    // a block's 32 loads of g and u are issued before its stores: the stores
    // may alias them as far as the compiler knows, so loads placed after a
    // store would each wait out a memory round trip (issuing them a block
    // ahead as well gained nothing more)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int f = tp.nt * NO + wn * WN + j * 32 + col_l;
        const bool fv = f < p.Nout;
        float gv[16], uv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t row = static_cast<uint32_t>(row_l + i * 32 + (r >> 2) * 8 + (r & 3));
          const uint32_t go = fv ? row * lg + static_cast<uint32_t>(f) * 4u : kStoreOOB;
          gv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, go, 0, kSaveLoadPolicy));
          uv[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, go + uoff_g, 0, kSaveLoadPolicy));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t row = static_cast<uint32_t>(row_l + i * 32 + (r >> 2) * 8 + (r & 3));
          const float g = gv[r], u = uv[r];
          const float dh = acc[i][j][r];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
          const float dg = dh * u * (sg * (1.0f + g * (1.0f - sg)));
          const float du = dh * (g * sg);
          const uint32_t co = fv ? row * ld + static_cast<uint32_t>(f) * 2u : kStoreOOB;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(dg), rc, co, 0, kHStorePolicy);
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(du), rc, co + uoff_c, 0, kHStorePolicy);
        }
      }
    return;
  }
  if (SWIGLU) {
    const uint16_t* base = static_cast<const uint16_t*>(p.C) + static_cast<int64_t>(tp.ti.row0) * p.ldc;
    const __amdgpu_buffer_rsrc_t rc = uniform_rsrc(base, static_cast<int64_t>(tp.ti.rows) * p.ldc * 2);
    const uint32_t ld = static_cast<uint32_t>(p.ldc) * 2u;  // bytes per row
    if (p.gu) {
      // training: keep g and u (fp32) for the backward's SwiGLU derivative
      const int64_t ldg = 2 * static_cast<int64_t>(p.Nout);
      const float* gbase = p.gu + static_cast<int64_t>(tp.ti.row0) * ldg;
      const __amdgpu_buffer_rsrc_t rg = uniform_rsrc(gbase, static_cast<int64_t>(tp.ti.rows) * ldg * 4);
      const uint32_t lg = static_cast<uint32_t>(ldg) * 4u, uoff = static_cast<uint32_t>(p.Nout) * 4u;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
          const int f = tp.nt * NO + wn * (WN / 2) + j * 32 + col_l;
          const uint32_t gb = f < p.Nout ? static_cast<uint32_t>(row_l * ldg + f) * 4u : kStoreOOB;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t off = gb + static_cast<uint32_t>(i * 32 + (r >> 2) * 8 + (r & 3)) * lg;
            const float g = acc[i][j][r], u = acc[i][j + NB / 2][r];
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g), rg, off, 0, kSaveStorePolicy);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(u), rg, off + uoff, 0, kSaveStorePolicy);
          }
        }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j) {
        const int f = tp.nt * NO + wn * (WN / 2) + j * 32 + col_l;
        const uint32_t cb = f < p.Nout ? static_cast<uint32_t>(row_l * p.ldc + f) * 2u : kStoreOOB;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // rows r and r + 1 are adjacent: one packed conversion, two stores
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          const bf16x2_t hv = {(__bf16)(silu_fast(acc[i][j][r]) * acc[i][j + NB / 2][r]),
                               (__bf16)(silu_fast(acc[i][j][r + 1]) * acc[i][j + NB / 2][r + 1])};
          const uint32_t bits = __builtin_bit_cast(uint32_t, hv);
          const uint32_t off = cb + static_cast<uint32_t>(i * 32 + (r >> 2) * 8 + (r & 3)) * ld;
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bits), rc, off, 0, kHStorePolicy);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bits >> 16), rc, off + ld, 0, kHStorePolicy);
        }
      }
  } else {
    const float* base = static_cast<const float*>(p.C) + tp.split * p.c_split_stride +
                        static_cast<int64_t>(tp.ti.row0) * p.ldc;
    const __amdgpu_buffer_rsrc_t rc = uniform_rsrc(base, static_cast<int64_t>(tp.ti.rows) * p.ldc * 4);
    const uint32_t ld = static_cast<uint32_t>(p.ldc) * 4u;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = tp.nt * NO + wn * WN + j * 32 + col_l;
        const uint32_t cb = n < p.Nout ? static_cast<uint32_t>(row_l * p.ldc + n) * 4u : kStoreOOB;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // the element goes through a scalar first: a bit_cast straight from
          // the vector subscript is compiled as element 0 for every r
          const float v = acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc,
                                                cb + static_cast<uint32_t>(i * 32 + (r >> 2) * 8 + (r & 3)) * ld, 0,
                                                CPOL);
        }
      }
  }
}

template <int MB, int NB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[MB][NB]) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// ---- buffer loads straight into LDS ------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `later` stages of LPS loads each are still in flight.
template <int LPS, int MAXLATER>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (MAXLATER >= 3) {
    if (later >= 3) { wait_vm<3 * LPS>(); return; }
  }
  if constexpr (MAXLATER >= 2) {
    if (later >= 2) { wait_vm<2 * LPS>(); return; }
  }
  if constexpr (MAXLATER >= 1) {
    if (later >= 1) { wait_vm<LPS>(); return; }
  }
  wait_vm<0>();
}

// LDS operations complete, then a workgroup barrier. The wait is the builtin
// (lgkmcnt 0, the other counters at their maximum) rather than inline asm, so
// the compiler's own wait insertion knows that every earlier LDS read has
// landed; the empty asm statements keep memory operations on their side.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One pipeline step: issue the loads of a later stage, then run the MFMAs of
// the current one. The restrict-qualified stage pointers tell the compiler the
// two stages are disjoint, so it does not hold the current stage's LDS reads
// until the just-issued loads land (the explicit waits and barrier at the top
// of each step order the stages).
template <int MB, int NB, class Issue, class Pipe>
__device__ __forceinline__ void dma_step(Issue& issue, bool do_issue, int kt_next, const uint16_t* __restrict__ a_cur,
                                         const uint16_t* __restrict__ b_cur, uint16_t* __restrict__ a_nxt,
                                         uint16_t* __restrict__ b_nxt, const int (&arow)[MB], const int (&brow)[NB],
                                         int khalf, f32x16_t (&acc)[MB][NB], int live, Pipe& fp) {
  if (do_issue) issue(a_nxt, b_nxt, kt_next);
  fp.stage(a_cur, b_cur, arow, brow, khalf, acc, live);
}

// LDS elements of one workgroup's operand stages.
template <int BM, int BN, int STAGES, int BK>
constexpr int dma_lds_elems() { return STAGES * (BM + BN) * BK; }

// The loads of one output tile: per-lane byte offsets of the tile's A and B
// rows and the wave-uniform buffer descriptors, and one K step's loads
// straight into an LDS stage.
//
// Lane q of 1-KB segment s holds row RPS*s + q/CPR at physical chunk q%CPR,
// which stores logical chunk (q%CPR) ^ key(row) (the swizzle is an XOR, so
// the same map in both directions). The key reads row bits 1..3, and every
// segment a wave fills starts at a row congruent to wave*RPS modulo 16, so
// one chunk per lane serves all of its loads.
template <int BM, int BN, int WGM, int WGN, int BK, bool SWIGLU, bool GATHER>
struct TileLoader {
  static constexpr int NW = WGM * WGN;
  static constexpr int CPR = BK / 8;                          // 16-byte chunks per LDS row
  static constexpr int RPS = 64 / CPR;                        // rows per 1-KB segment (one load per wave)
  static constexpr int IA = BM / RPS / NW, IB = BN / RPS / NW;  // segments a wave fills per stage
  static constexpr int LPS = IA + IB;
  static constexpr int NO = SWIGLU ? BN / 2 : BN;
  // B segment of load i: for swiglu the first IB/2 loads of every wave fill
  // gate rows [0, BN/2) and the rest the matching up rows, so the weight
  // matrix of each load is known at compile time
  static constexpr int IBH = SWIGLU ? IB / 2 : IB;
  static_assert(IA * NW * RPS == BM && IB * NW * RPS == BN, "segments must divide among waves");
  static_assert((NW * RPS) % 16 == 0 && (BN / 2) % 16 == 0, "segment rows must keep the swizzle key");
  static_assert(!SWIGLU || IB % 2 == 0, "swiglu splits the B loads in halves");

  uint32_t aoff[IA], boff[IB];
  __amdgpu_buffer_rsrc_t ra, rb0, rb1;
  int wave, lchunk, kb0, kb1;

  __device__ __forceinline__ void init(const GemmParams& p, const TilePos& tp) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lrow = lane / CPR;
    lchunk = (lane % CPR) ^ swz_key<BK>(wave * RPS + lrow);
    kb0 = tp.kb0;
    kb1 = tp.kb1;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int r = (i * NW + wave) * RPS + lrow;
      const bool v = r < tp.ti.rows;
      int src = tp.ti.row0 + r;
      if (GATHER) src = v ? p.row_token[src] : 0;
      aoff[i] = v ? static_cast<uint32_t>(src) * static_cast<uint32_t>(p.lda) * 2u + lchunk * 16u : kOOB;
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int r = ((i % IBH) * NW + wave) * RPS + lrow;  // row within the gate (or plain) block
      const int f = tp.nt * NO + r;
      boff[i] = f < p.Nout ? static_cast<uint32_t>(f) * static_cast<uint32_t>(p.ldb) * 2u + lchunk * 16u : kOOB;
    }
    const int64_t b_bytes = static_cast<int64_t>(p.Nout) * p.ldb * 2;
    ra = uniform_rsrc(p.A, p.a_rows * p.lda * 2);
    const uint16_t* b0 = static_cast<const uint16_t*>(p.B0) + tp.ti.expert * p.b_expert_stride;
    const uint16_t* b1 = SWIGLU ? static_cast<const uint16_t*>(p.B1) + tp.ti.expert * p.b_expert_stride : b0;
    rb0 = uniform_rsrc(b0, b_bytes);
    rb1 = uniform_rsrc(b1, b_bytes);
  }

  // K step kt's A rows into the LDS stage at a_dst
  __device__ __forceinline__ void issue_a(uint16_t* a_dst, int kt) const {
    const int kb = kb0 + kt * BK;
    const bool kval = kb + lchunk * 8 < kb1;
    const uint32_t kbyte = static_cast<uint32_t>(kb) * 2u;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const uint32_t vo = (kval && aoff[i] != kOOB) ? aoff[i] + kbyte : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(a_dst + (i * NW + wave) * 512), 16, vo, 0, 0, 0);
    }
  }

  // K step kt's B rows into the LDS stage at b_dst
  __device__ __forceinline__ void issue_b(uint16_t* b_dst, int kt) const {
    const int kb = kb0 + kt * BK;
    const bool kval = kb + lchunk * 8 < kb1;
    const uint32_t kbyte = static_cast<uint32_t>(kb) * 2u;
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const uint32_t vo = (kval && boff[i] != kOOB) ? boff[i] + kbyte : kOOB;
      const int seg = (i % IBH) * NW + wave + (i >= IBH ? (BN / 2 / RPS) : 0);
      if (i < IBH)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb0, (lds_ptr_t)(b_dst + seg * 512), 16, vo, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb1, (lds_ptr_t)(b_dst + seg * 512), 16, vo, 0, 0, 0);
    }
  }
};

// One KN operand's loads: BK rows x 256 columns per stage, 2 rows per 1-KB
// segment, NW waves each filling BK / 2 / NW segments. Lane q of a segment
// holds row q / 32 at physical chunk q % 32, i.e. logical chunk
// (q % 32) ^ (4 (row & 3)); row & 3 is the same for every segment of a wave,
// so one column offset per lane serves all of its loads.
//   rows: K row k reads source row k (plain), map[k] (gather), or for a
//   split operand row k of src0 when k < ksplit and row k - ksplit of src1
//   (ksplit even, so both rows of a segment come from one source).
// Gather: the 64 map entries of a K step go into a two-slot LDS ring with one
// direct-to-LDS load by wave 0, a step ahead (so no vector register waits on
// a map load, and the compiler places no wait on the stage loads before the
// MFMAs). Step kt reads slot kt & 1; the load for step kt + 1 overwrites the
// slot of step kt - 1, which every wave read before the barrier of the step
// in which it is issued.
template <int NW, int BK, bool GATHER>
struct KnOperand {
  static constexpr int I = BK / 2 / NW;  // segments a wave fills per stage
  static_assert(I * 2 * NW == BK, "KN segments must divide among waves");
  static_assert(!GATHER || BK == 64, "a map ring slot holds one 64-row K step");
  __amdgpu_buffer_rsrc_t r0, r1, rmap;
  uint32_t colb;     // this lane's byte offset within a row, or kOOB (columns past the extent)
  uint32_t ldbytes;  // bytes per source row
  int wave, half, kb1, ksplit;
  int* ring;         // gather: [2][64] source rows of K steps (LDS)

  __device__ __forceinline__ void init(const void* src0, const void* src1, int64_t src_rows, int64_t ld, int col0,
                                       int cols, int kend, int ksplit_, const int32_t* map, int* ring_) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    half = lane >> 5;
    const int key = ((2 * wave + half) & 3) << 2;
    const int c = (lane & 31) ^ key;
    colb = c * 8 < cols ? static_cast<uint32_t>(col0 + c * 8) * 2u : kOOB;
    ldbytes = static_cast<uint32_t>(ld) * 2u;
    kb1 = kend;
    ksplit = ksplit_;
    ring = ring_;
    r0 = uniform_rsrc(src0, src_rows * ld * 2);
    r1 = uniform_rsrc(src1 ? src1 : src0, src_rows * ld * 2);
    if constexpr (GATHER) rmap = uniform_rsrc(map, static_cast<int64_t>(kend) * 4);  // map[k] reads 0 for k >= kend
  }

  __device__ __forceinline__ int row(int s, int kb) const { return kb + 2 * s + half; }

  // gather: wave 0 loads the map entries of the K step at kb into ring slot
  // `slot` (entries past the K range read as 0)
  __device__ __forceinline__ void fetch(int kb, int slot) const {
    if constexpr (GATHER) {
      if (wave == 0) {
        const uint32_t vo = static_cast<uint32_t>(kb + (threadIdx.x & 63)) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rmap, (lds_ptr_t)(ring + slot * 64), 4, vo, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void issue(uint16_t* dst, int kb, int slot) const {
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int s = i * NW + wave;
      const int k = row(s, kb);
      const bool second = kb + 2 * s >= ksplit;  // wave-uniform
      int src;
      // an LDS read (the address space said explicitly, so it is no flat load)
      if constexpr (GATHER) src = ((__attribute__((address_space(3))) const int*)ring)[slot * 64 + 2 * s + half];
      else src = second ? k - ksplit : k;
      const uint32_t vo = (k < kb1 && colb != kOOB) ? static_cast<uint32_t>(src) * ldbytes + colb : kOOB;
      if (second)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, (lds_ptr_t)(dst + s * 512), 16, vo, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, (lds_ptr_t)(dst + s * 512), 16, vo, 0, 0, 0);
    }
  }
};

// The backward's tile loads. LAY 1 (input gradients): A is the usual
// K-contiguous row operand (dE, or dg | du, rows of the tile's expert); B is
// KN, the expert's weights, split at g.ksplit between B0 and B1 (Wgate and
// Wup). LAY 2 (weight gradients): both KN over the expert's rows
// [kb0, kb1) of the permuted order; A's columns are the tile's M rows
// (ti.row0 .. + ti.rows), B's the tile's N columns; B rows are gathered
// through row_token when it is set (x for dWgate and dWup).
template <int BM, int BN, int WGM, int WGN, int BK, int LAY, bool BGATHER>
struct BwdLoader {
  static constexpr int NW = WGM * WGN;
  static_assert(BM == kKnCols && BN == kKnCols, "KN stages hold 256 columns");
  using Tn = TileLoader<BM, BN, WGM, WGN, BK, false, false>;
  using KnA = KnOperand<NW, BK, false>;
  using KnB = KnOperand<NW, BK, BGATHER>;
  static constexpr int LPS = (LAY == 1 ? Tn::IA : KnA::I) + KnB::I;
  static constexpr int NO = BN;
  Tn ta;
  KnA ka;
  KnB kb;
  int kb0;

  // ring: BGATHER's map ring ([2][64] int32 of LDS, not used otherwise). With
  // BGATHER, init loads the first K step's map entries and waits for them at
  // a workgroup barrier, so every wave must call it.
  __device__ __forceinline__ void init(const GemmParams& p, const TilePos& tp, int* ring = nullptr) {
    kb0 = tp.kb0;
    if constexpr (LAY == 1) {
      ta.init(p, tp);  // its A rows; its B part is not used
      const uint16_t* b0 = static_cast<const uint16_t*>(p.B0) + tp.ti.expert * p.b_expert_stride;
      const uint16_t* b1 = p.B1 ? static_cast<const uint16_t*>(p.B1) + tp.ti.expert * p.b_expert_stride : b0;
      kb.init(b0, b1, p.b_rows, p.ldb, tp.nt * BN, p.Nout - tp.nt * BN, tp.kb1, p.ksplit, nullptr, nullptr);
    } else {
      ka.init(p.A, nullptr, p.a_rows, p.lda, tp.ti.row0, tp.ti.rows, tp.kb1, 1 << 30, nullptr, nullptr);
      kb.init(p.B0, nullptr, p.b_rows, p.ldb, tp.nt * BN, p.Nout - tp.nt * BN, tp.kb1, 1 << 30, p.row_token, ring);
      if constexpr (BGATHER) {
        kb.fetch(kb0, 0);
        wait_vm<0>();
        __syncthreads();
      }
    }
  }

  __device__ __forceinline__ void issue_a(uint16_t* a_dst, int kt) {
    if constexpr (LAY == 1) ta.issue_a(a_dst, kt);
    else ka.issue(a_dst, kb0 + kt * BK, 0);
  }
  // K step kt's B rows; with BGATHER, also the map entries of step kt + 1
  // (steps are issued in order, one per K step)
  __device__ __forceinline__ void issue_b(uint16_t* b_dst, int kt) {
    kb.issue(b_dst, kb0 + kt * BK, kt & 1);
    if constexpr (BGATHER) kb.fetch(kb0 + (kt + 1) * BK, (kt + 1) & 1);
  }
};

// LDS stage addresses of the operand stages in `smem`.
template <int BM, int BN, int BK>
__device__ __forceinline__ uint16_t* stage_a(uint16_t* smem, int st) { return smem + st * (BM + BN) * BK; }
template <int BM, int BN, int BK>
__device__ __forceinline__ uint16_t* stage_b(uint16_t* smem, int st) { return smem + st * (BM + BN) * BK + BM * BK; }

// Nothing to do during or after the K loop.
struct NoHook {
  __device__ __forceinline__ void operator()(uint16_t*, uint16_t*, int) const {}
};
struct NoReserve {
  __device__ __forceinline__ void operator()() const {}
};

// One output tile with buffer loads straight into LDS: the operand stages
// live in `smem` (dma_lds_elems elements, one LDS object). The caller makes
// sure no wave still reads `smem` from an earlier tile.
//
// K step kt uses stage buffer (sbase + kt) % STAGES. pre says how much of
// step 0 an earlier call already issued into buffer sbase: 0 nothing, 1 the B
// rows, 2 A and B. reserve() runs three K steps before the end (at step 0 of
// a shorter tile); after the MFMAs of the last K step are issued, hook(a, b,
// buf) may issue loads into stage buffer buf (at a, b), which no wave reads
// any more; the epilogue follows.
//
// LAY 0: both operands K-contiguous (the forward); LAY 1 and 2: the
// backward's K-outer operands (BwdLoader), B (LAY 1) or both (LAY 2) staged
// as KN and read with the transposing LDS reads; BGATHER gathers LAY 2's B
// rows through row_token.
template <int BM, int BN, int WGM, int WGN, int STAGES, int BK, bool SWIGLU, bool GATHER, class Hook = NoHook,
          class Reserve = NoReserve, int LAY = 0, bool BGATHER = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const TilePos& tp, uint16_t* smem, int sbase = 0,
                                          int pre = 0, Hook&& hook = Hook{}, Reserve&& reserve = Reserve{},
                                          bool poison = false) {
  static_assert(LAY == 0 || (!SWIGLU && !GATHER && BK == 64), "the backward's tiles are plain");
  using Loader = std::conditional_t<LAY == 0, TileLoader<BM, BN, WGM, WGN, BK, SWIGLU, GATHER>,
                                    BwdLoader<BM, BN, WGM, WGN, BK, LAY, BGATHER>>;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int LPS = Loader::LPS;
  constexpr int NO = Loader::NO;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!SWIGLU || NB % 2 == 0, "swiglu needs gate/up block pairs");
  static_assert(STAGES >= 2 && STAGES <= 5 && (STAGES - 2) * LPS <= 63, "stage count");

  auto sA = [&](int st) { return stage_a<BM, BN, BK>(smem, st); };
  auto sB = [&](int st) { return stage_b<BM, BN, BK>(smem, st); };

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave w takes row group w % WGM and column group w / WGM: the waves that
  // share a SIMD (w and w + 4) cover different column groups, so a tile whose
  // last columns lie past Nout still gives every SIMD the same MFMA work
  const int wm = wave % WGM, wn = wave / WGM;

  Loader ld;
  if constexpr (LAY == 0) ld.init(p, tp);
  else ld.init(p, tp, reinterpret_cast<int*>(smem + dma_lds_elems<BM, BN, STAGES, BK>()));
  auto issue = [&](uint16_t* a_dst, uint16_t* b_dst, int kt) {
    ld.issue_a(a_dst, kt);
    ld.issue_b(b_dst, kt);
  };

  f32x16_t acc[MB][NB];
  zero_acc(acc);
  int arow[MB], brow[NB];
  frag_rows<WM, WN, MB, NB, BN, SWIGLU>(wm, wn, lane, arow, brow);
  if constexpr (LAY == 2) {
#pragma unroll
    for (int i = 0; i < MB; ++i) arow[i] = kn_frag_off(wm * WM + i * 32, lane);
  }
  if constexpr (LAY >= 1) {
#pragma unroll
    for (int j = 0; j < NB; ++j) brow[j] = kn_frag_off(wn * WN + j * 32, lane);
  }
  const int khalf = lane >> 5;
  // 32-row blocks of this wave that hold rows of the tile; none when all of
  // the wave's output columns lie past Nout (an expert's last column tile)
  const bool cols_dead = tp.nt * NO + wn * (SWIGLU ? WN / 2 : WN) >= p.Nout;
  const int live =
      cols_dead ? 0 : __builtin_amdgcn_readfirstlane(max(0, min(MB, (tp.ti.rows - wm * WM + 31) / 32)));

  if (tp.KT > 0) {
    if (pre < 2) ld.issue_a(sA(sbase), 0);
    if (pre < 1) ld.issue_b(sB(sbase), 0);
  }
#pragma unroll
  for (int s = 1; s < STAGES - 1; ++s)
    if (s < tp.KT) issue(sA((sbase + s) % STAGES), sB((sbase + s) % STAGES), s);
  // the K loop, in a branch-free copy for full tiles and one that skips a
  // partly filled tile's empty row blocks
  const int kt_reserve = max(0, tp.KT - 3);
  auto kloop = [&](auto partial) {
    FragPipe<MB, NB, BK, decltype(partial)::value, LAY == 2, LAY >= 1> fp;
    fp.init();
    for (int kt = 0; kt < tp.KT; ++kt) {
      const int later = min(STAGES - 2, tp.KT - 1 - kt);
      wait_stage<LPS, STAGES - 2>(later);
      lds_barrier();  // stage kt is complete for every wave; stage kt-1 is free
      if (kt == kt_reserve) reserve();
      const int st = (sbase + kt) % STAGES, nx = (sbase + kt + STAGES - 1) % STAGES;
      dma_step<MB, NB>(issue, kt + STAGES - 1 < tp.KT, kt + STAGES - 1, sA(st), sB(st), sA(nx), sB(nx), arow, brow,
                       khalf, acc, live, fp);
    }
    fp.mma(1, acc, live);  // the last stage's last slice
  };
  if (live == MB)
    kloop(std::false_type{});
  else
    kloop(std::true_type{});
  const int fb = (sbase + tp.KT) % STAGES;
  hook(sA(fb), sB(fb), fb);
  if (poison) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_nanf("");
  }
  epilogue<WM, WN, MB, NB, SWIGLU, LAY == 2 ? kGradStorePolicy : kYStorePolicy>(p, tp, wm, wn, lane, NO, acc);
}

// ---- decode-shaped tiles: a long K step per weight row -----------------------
//
// When experts get few rows, the GEMMs stream the expert weights from HBM
// once and the matrix cores are nearly idle, so the tile is shaped for the
// memory system: 32 rows of A, 64 rows of B (32 gate and 32 up rows for
// swiglu) and a K step of BK = 128 bf16, 256 contiguous bytes of every weight
// row per step, in three stages of 24 KB, so that two workgroups share a
// compute unit and one's barrier wait overlaps the other's loads. The NW
// waves split each step's K slices; their partial sums meet in LDS after the
// K loop and wave 0 runs the epilogue.
//
// LDS rows hold BK bf16 (16 or 32 chunks of 16 bytes); chunk c of row r sits
// at physical chunk c ^ (r & 15), so the 16 rows an MFMA operand read covers
// at one chunk land in 16 distinct groups of four banks.
constexpr int kDecBM = 32, kDecBN = 64;

template <int BK>
__device__ __forceinline__ int dec_swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 15)) << 3);
}

template <int BM, int BK, int STAGES, int NW, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(NW * 64) void k_gemm_decode(GemmParams p) {
  constexpr int BN = kDecBN, MB = BM / 32;
  constexpr int NO = SWIGLU ? BN / 2 : BN;
  constexpr int CPR = BK / 8;              // 16-byte chunks per LDS row
  constexpr int RPS = 64 / CPR;            // rows per 1-KB load segment (one load per wave)
  constexpr int IA = BM / RPS / NW, IB = BN / RPS / NW;  // segments a wave fills per stage
  constexpr int LPS = IA + IB;
  constexpr int KS = BK / 16;              // MFMA K slices per step
  constexpr int KSW = KS / NW;             // slices per wave
  static_assert(CPR >= 16 && IA * RPS * NW == BM && IB * RPS * NW == BN && KSW * NW == KS, "decode tile shape");
  static_assert(STAGES >= 2 && (STAGES - 2) * LPS <= 63, "stage count");
  static_assert(STAGES * (BM + BN) * BK >= NW * MB * 2 * 16 * 64 * 2, "partials fit in the stages");
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * (BM + BN) * BK];

  TilePos tp;
  if (!decode_tile<BM, NO, BK>(p, tp)) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // per-load lane offsets: segment i * NW + wave, row RPS * segment + lane / CPR,
  // physical chunk lane % CPR holding logical chunk (lane % CPR) ^ (row & 15)
  const int prow = lane / CPR, pchunk = lane % CPR;
  uint32_t aoff[IA], boff[IB];
  int alc[IA], blc[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r = (i * NW + wave) * RPS + prow;
    alc[i] = pchunk ^ (r & 15);
    const bool v = r < tp.ti.rows;
    int src = tp.ti.row0 + r;
    if (GATHER) src = v ? p.row_token[src] : 0;
    aoff[i] = v ? static_cast<uint32_t>(src) * static_cast<uint32_t>(p.lda) * 2u + alc[i] * 16u : kOOB;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int r = (i * NW + wave) * RPS + prow;  // B row of the tile
    blc[i] = pchunk ^ (r & 15);
    const int f = tp.nt * NO + (SWIGLU && r >= BN / 2 ? r - BN / 2 : r);
    boff[i] = f < p.Nout ? static_cast<uint32_t>(f) * static_cast<uint32_t>(p.ldb) * 2u + blc[i] * 16u : kOOB;
  }
  const int64_t b_bytes = static_cast<int64_t>(p.Nout) * p.ldb * 2;
  const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(p.A, p.a_rows * p.lda * 2);
  const uint16_t* b0 = static_cast<const uint16_t*>(p.B0) + tp.ti.expert * p.b_expert_stride;
  const uint16_t* b1 = SWIGLU ? static_cast<const uint16_t*>(p.B1) + tp.ti.expert * p.b_expert_stride : b0;
  const __amdgpu_buffer_rsrc_t rb0 = uniform_rsrc(b0, b_bytes), rb1 = uniform_rsrc(b1, b_bytes);

  auto sA = [&](int st) { return smem + st * (BM + BN) * BK; };
  auto sB = [&](int st) { return smem + st * (BM + BN) * BK + BM * BK; };
  auto issue = [&](int st, int kt) {
    const int kb = tp.kb0 + kt * BK;
    const uint32_t kbyte = static_cast<uint32_t>(kb) * 2u;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const bool kval = kb + alc[i] * 8 < tp.kb1;
      const uint32_t vo = (kval && aoff[i] != kOOB) ? aoff[i] + kbyte : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(sA(st) + (i * NW + wave) * 512), 16, vo, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int r0 = (i * NW + wave) * RPS;  // first row of the segment (wave-uniform)
      const bool kval = kb + blc[i] * 8 < tp.kb1;
      const uint32_t vo = (kval && boff[i] != kOOB) ? boff[i] + kbyte : kOOB;
      if (!SWIGLU || r0 < BN / 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb0, (lds_ptr_t)(sB(st) + (i * NW + wave) * 512), 16, vo, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb1, (lds_ptr_t)(sB(st) + (i * NW + wave) * 512), 16, vo, 0, 0, 0);
    }
  };

  f32x16_t acc[MB][2];
  zero_acc(acc);
  const int frow = lane & 31, khalf = lane >> 5;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < tp.KT) issue(s, s);
  for (int kt = 0; kt < tp.KT; ++kt) {
    wait_stage<LPS, STAGES - 2>(min(STAGES - 2, tp.KT - 1 - kt));
    lds_barrier();  // stage kt is complete for every wave; stage kt-1 is free
    if (kt + STAGES - 1 < tp.KT) issue((kt + STAGES - 1) % STAGES, kt + STAGES - 1);
    const uint16_t* a = sA(kt % STAGES);
    const uint16_t* b = sB(kt % STAGES);
    bf16x8_t af[KSW][MB], bf0[KSW], bf1[KSW];
#pragma unroll
    for (int q = 0; q < KSW; ++q) {
      const int chunk = (wave * KSW + q) * 2 + khalf;
#pragma unroll
      for (int i = 0; i < MB; ++i) af[q][i] = *reinterpret_cast<const bf16x8_t*>(&a[dec_swz<BK>(i * 32 + frow, chunk)]);
      bf0[q] = *reinterpret_cast<const bf16x8_t*>(&b[dec_swz<BK>(frow, chunk)]);
      bf1[q] = *reinterpret_cast<const bf16x8_t*>(&b[dec_swz<BK>(32 + frow, chunk)]);
    }
#pragma unroll
    for (int q = 0; q < KSW; ++q)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[q][i], bf0[q], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[q][i], bf1[q], acc[i][1], 0, 0, 0);
      }
  }

  // partial sums of the four waves, added in wave order by wave 0
  lds_barrier();
  float* red = reinterpret_cast<float*>(smem);  // [wave][i][j][r][lane]
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[i][j][r];
        red[(((wave * MB + i) * 2 + j) * 16 + r) * 64 + lane] = v;
      }
  lds_barrier();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = red[((i * 2 + j) * 16 + r) * 64 + lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[(((w * MB + i) * 2 + j) * 16 + r) * 64 + lane];
        acc[i][j][r] = v;
      }
  epilogue<BM, BN, MB, 2, SWIGLU>(p, tp, 0, 0, lane, NO, acc);
}

// ---- both expert GEMMs in one persistent launch ---------------------------------
//
// A row block is BM consecutive permuted rows of one expert. The gate/up
// GEMM of a row block is NT1 tiles (one per 128-column slice of h); its down
// projection is NT2 tiles, and those read every column of the row block's h,
// so they may start only once all NT1 gate/up tiles of that row block are
// done. Workgroups stay resident and take work items from one queue in
// ticket order: first every gate/up tile (expert by expert, a group of the
// expert's row blocks at a time), then the down tiles in row-block order, so
// the down tiles of the first row blocks fill the compute units that the last
// round of gate/up tiles leaves idle. Workgroup b's first ticket is b, and
// the first tickets are remapped as blockIdx would be: workgroups are dealt
// round-robin to the 8 XCDs, so the first round's tiles that share weight
// panels land on one XCD and its L2; the queue then hands out tickets from
// the grid size on. A down tile waits, with a bounded spin,
// on its row block's count of finished gate/up tiles; all gate/up tickets
// come before any down ticket, so every tile it waits on is already running
// in, or reserved by, a workgroup that waits on nothing, and the wait always
// ends.

constexpr int kSchedTicket = 0;     // sched[kSchedTicket]: next ticket
constexpr int kSchedError = 8;      // sched[kSchedError] = 1 if a wait gave up
constexpr int kSchedDone = 16;      // sched[kSchedDone + rb]: finished gate/up tiles of row block rb
constexpr int kFusedBM = 256, kFusedBN = 256;

// Row block rb's expert and rows (lane e holds expert e's segment and its
// inclusive prefix count of row blocks).
template <int BM>
__device__ __forceinline__ TileInfo row_block(int rb, int eoff, int ecnt, int etl, int incl) {
  const int e = __popcll(__ballot(incl <= rb));
  const int local = rb - __shfl(incl - etl, e, 64);
  TileInfo ti;
  ti.expert = __builtin_amdgcn_readfirstlane(e);
  ti.row0 = __builtin_amdgcn_readfirstlane(__shfl(eoff, e, 64) + local * BM);
  ti.rows = __builtin_amdgcn_readfirstlane(min(BM, __shfl(ecnt, e, 64) - local * BM));
  return ti;
}

// Spin until *ctr reaches target, at most `limit` polls; returns false (and
// raises the error word) when it gives up. The loads are relaxed: an acquire
// load invalidates the caches every time round the loop, under the tiles that
// run beside it; the caller issues one acquire fence after the wait.
__device__ __forceinline__ bool wait_count(int32_t* ctr, int target, int32_t* err, int limit) {
  for (int it = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++it) {
    if (it >= limit) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  return true;
}

// G1_SWIGLU: g1 is the gate/up GEMM with the SwiGLU epilogue (the forward);
// otherwise g1 is a plain GEMM whose epilogue is g1.epi (the backward's dh
// with the SwiGLU derivative), and g2 reads its output the same way.
template <int BM, int BN, int WGM, int WGN, int STAGES, int BK, bool GATHER, bool G1_SWIGLU>
__global__ __launch_bounds__(WGM * WGN * 64) void k_experts_fused(FusedParams fp) {
  constexpr int kElems = dma_lds_elems<BM, BN, STAGES, BK>();
  // the operand stages and, after them, the broadcast work item: one LDS object
  __shared__ __attribute__((aligned(16))) uint16_t smem[kElems + 8];
  int* s_item = reinterpret_cast<int*>(smem + kElems);  // [0] next ticket, [1] a down tile's wait gave up
  constexpr int GM = 8;  // most row blocks per group of gate/up tiles
  const GemmParams& g1 = fp.g1;
  const GemmParams& g2 = fp.g2;
  const int lane = threadIdx.x & 63;
  // the forward's operands are K-contiguous; the backward's weights are KN
  constexpr int LAY = G1_SWIGLU ? 0 : 1;
  using Loader1 = std::conditional_t<LAY == 0, TileLoader<BM, BN, WGM, WGN, BK, G1_SWIGLU, GATHER>,
                                     BwdLoader<BM, BN, WGM, WGN, BK, 1, false>>;
  using Loader2 = std::conditional_t<LAY == 0, TileLoader<BM, BN, WGM, WGN, BK, false, false>,
                                     BwdLoader<BM, BN, WGM, WGN, BK, 1, false>>;

  // per-expert row blocks (lane e = expert e), inclusive scan over lanes
  // (clamped to the rows the workspace holds, so RB never exceeds the row
  // blocks the queue counters were sized for)
  int eoff = 0, ecnt = 0;
  expert_segment_wave(g1.offsets, g1.N, static_cast<int>(g1.rows_max), eoff, ecnt, g1.dbg);
  const int etl = (ecnt + BM - 1) / BM;
  int incl = etl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  // the segments do not overlap and hold at most rows_max rows, so RB stays
  // within the ceil(rows_max / BM) + N row blocks the queue counters hold
  const int RB = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
  const int NT1 = G1_SWIGLU ? (g1.Nout + BN / 2 - 1) / (BN / 2) : (g1.Nout + BN - 1) / BN;
  const int NT2 = (g2.Nout + BN - 1) / BN;
  const int n1 = RB * NT1, n2 = RB * NT2;
  const int G = gridDim.x;
  const int S = min(n1, G);  // tickets below S are remapped XCD-aware
  // the backward's third GEMM (tiles that never wait): P of its n3 tiles go
  // right after the g1 tiles, to keep the compute units that the first round
  // of g1 tiles leaves free busy until those finish (about (G - n1) units, each
  // for a g1 tile's K steps over a g3 tile's), and the rest after the g2
  // tiles, where they fill the last round
  constexpr bool W3 = !G1_SWIGLU;
  int n3 = 0, P = 0, mt3 = 0, nt3 = 0;
  if constexpr (W3) {
    if (fp.g3.N > 0) {
      mt3 = (fp.m3 + BM - 1) / BM;
      nt3 = (fp.g3.Nout + BN - 1) / BN;
      n3 = mt3 * nt3 * fp.g3.N;
      const int kt1 = (g1.K + BK - 1) / BK;
      const int kt3 = max(1, static_cast<int>((fp.g3.rows_max / max(1, fp.g3.N) + BK - 1) / BK));
      P = min(n3, max(0, G - n1) * max(1, kt1 / kt3));
    }
  }
  const int ntot = n1 + n2 + n3;

  // tile of ticket t: 0 a gate/up (g1) tile, 1 a down (g2) tile, 2 a g3 tile;
  // its row block (types 0 and 1) and position
  auto decode = [&](int t, TilePos& tp, int& rb) {
    const int it = t < S ? xcd_remap(t, S) : t;
    tp = TilePos{};
    if (W3 && n3 > 0 && (it >= n1 + P + n2 || (it >= n1 && it < n1 + P))) {
      // g3 tile j: expert e, four M tiles at a time with the N tile fastest
      const int j = it < n1 + P ? it - n1 : it - n1 - n2;
      constexpr int GM3 = 4;
      const int per_e = mt3 * nt3;
      const int e = j / per_e;
      const int q = j - e * per_e;
      const int g = q / (GM3 * nt3);
      const int gm = min(GM3, mt3 - g * GM3);
      const int rq = q - g * GM3 * nt3;
      const int mt = g * GM3 + rq % gm;
      tp.nt = __builtin_amdgcn_readfirstlane(rq / gm);
      tp.ti.expert = 0;
      tp.ti.row0 = __builtin_amdgcn_readfirstlane(mt * BM);
      tp.ti.rows = __builtin_amdgcn_readfirstlane(min(BM, fp.m3 - mt * BM));
      tp.split = __builtin_amdgcn_readfirstlane(e);
      const int off = __builtin_amdgcn_readfirstlane(__shfl(eoff, e, 64));
      const int cnt = __builtin_amdgcn_readfirstlane(__shfl(ecnt, e, 64));
      tp.kb0 = off;
      tp.kb1 = off + cnt;
      tp.KT = (cnt + BK - 1) / BK;
      rb = -1;
      return 2;
    }
    const int it2 = (W3 && it >= n1 + P) ? it - P : it;  // g1 and g2 tickets without the first g3 tiles
    if (it2 < n1) {
      // gate/up tiles go expert by expert, in groups of at most GM of the
      // expert's row blocks (split evenly), column tile by column tile with the
      // row block fastest: the tiles of a group share their weight panels, and
      // an expert's last, partly filled row block rides along with the others
      const int e = __popcll(__ballot(incl * NT1 <= it2));  // expert of the tile
      const int rb0 = __builtin_amdgcn_readfirstlane(__shfl(incl - etl, e, 64));
      const int R = __builtin_amdgcn_readfirstlane(__shfl(etl, e, 64));
      const int ng = (R + GM - 1) / GM, base = R / ng, extra = R % ng;
      int q = it2 - rb0 * NT1;  // tile within the expert
      int g0 = 0, gm = base + (extra > 0 ? 1 : 0);
      for (int g = 0; q >= gm * NT1; ++g) {  // find the group (ng is small)
        q -= gm * NT1;
        g0 += gm;
        gm = base + (g + 1 < extra ? 1 : 0);
      }
      rb = rb0 + g0 + q % gm;
      tp.nt = q / gm;
      tp.ti = row_block<BM>(rb, eoff, ecnt, etl, incl);
      tp.kb1 = g1.K;
      tp.KT = (g1.K + BK - 1) / BK;
      return 0;
    }
    const int j = it2 - n1;
    rb = j / NT2;
    tp.nt = j % NT2;
    tp.ti = row_block<BM>(rb, eoff, ecnt, etl, incl);
    tp.kb1 = g2.K;
    tp.KT = (g2.K + BK - 1) / BK;
    return 1;
  };

  // the first round's tickets are the workgroups' own indices (workgroup b
  // runs on XCD b % 8, which the remap of the first S tickets relies on; an
  // atomic draw would hand them out in whatever order the XCDs arrive); the
  // queue hands out the tickets from G on
  int ticket = static_cast<int>(blockIdx.x);
  int sbase = 0, pre = 0;  // stage buffer of K step 0, and how much of it is already loading
  while (ticket < ntot) {
    // The next ticket is reserved three K steps before this tile ends (late
    // enough that the queue still balances the tail, early enough that the
    // atomic's latency hides); it reaches the workgroup after the K loop,
    // where the hook issues the next tile's first stage into the free stage
    // buffer: all of it for a gate/up (or g3) tile, only the weights for a
    // down tile, whose h rows may not be ready. Every gate/up ticket is
    // smaller than every down ticket, g3 tiles wait on nothing, and a
    // workgroup reserves its next ticket only after its own wait: so a
    // workgroup that waits in a down tile holds no other ticket, and every
    // gate/up ticket still runs in or is reserved by a workgroup that waits on
    // nothing (a first-round gate/up ticket belongs to a workgroup of smaller
    // index than any first-round down ticket's, dispatched before it).
    int reserved = ntot;  // "none" unless reserve() runs
    auto reserve = [&]() {
      if (threadIdx.x == 0) reserved = G + atomicAdd(&fp.sched[kSchedTicket], 1);
    };
    int next = ntot, nsbase = 0, npre = 0;
    auto hook = [&](uint16_t* a_free, uint16_t* b_free, int fb) {
      if (threadIdx.x == 0) *s_item = reserved;
      __syncthreads();
      next = __builtin_amdgcn_readfirstlane(*s_item);
      if (next < ntot) {
        TilePos tq;
        int rq;
        const int ty = decode(next, tq, rq);
        if (ty == 0) {
          Loader1 lq;
          lq.init(g1, tq);
          lq.issue_a(a_free, 0);
          lq.issue_b(b_free, 0);
          npre = 2;
        } else if (ty == 1) {
          Loader2 lq;
          lq.init(g2, tq);
          lq.issue_b(b_free, 0);
          npre = 1;
        } else if constexpr (W3) {
          BwdLoader<BM, BN, WGM, WGN, BK, 2, false> lq;
          lq.init(fp.g3, tq);
          lq.issue_a(a_free, 0);
          lq.issue_b(b_free, 0);
          npre = 2;
        }
        nsbase = fb;
      }
    };
    TilePos tp;
    int rb;
    const int ty = decode(ticket, tp, rb);
    if (W3 && ty == 2) {
      if constexpr (W3)
        gemm_tile<BM, BN, WGM, WGN, STAGES, BK, false, false, decltype(hook)&, decltype(reserve)&, 2>(
            fp.g3, tp, smem, sbase, pre, hook, reserve);
    } else if (ty == 0) {
      gemm_tile<BM, BN, WGM, WGN, STAGES, BK, G1_SWIGLU, GATHER, decltype(hook)&, decltype(reserve)&, LAY>(
          g1, tp, smem, sbase, pre, hook, reserve);
      // publish: every wave waits until its device-scope h stores have
      // completed (the wait also covers the next tile's first loads, issued
      // before the epilogue and needed next anyway), then one count. No L2
      // write-back: the h lines were written through at device scope.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); the other counters at their maximum
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&fp.sched[kSchedDone + rb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // a wait that gives up leaves the error word raised and writes NaN over
      // this tile's outputs instead of sums of h rows that may be unpublished
      if (threadIdx.x == 0) {
        const bool ok = wait_count(&fp.sched[kSchedDone + rb], NT1 + fp.wait_extra, &fp.sched[kSchedError],
                                   fp.spin_limit);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_item[1] = ok ? 0 : 1;
      }
      __syncthreads();
      const bool poison = __builtin_amdgcn_readfirstlane(s_item[1]) != 0;
      gemm_tile<BM, BN, WGM, WGN, STAGES, BK, false, false, decltype(hook)&, decltype(reserve)&, LAY>(
          g2, tp, smem, sbase, pre, hook, reserve, poison);
    }
    ticket = next;
    sbase = nsbase;
    pre = npre;
  }
  // the workgroup that drew the first ticket past the end reduces the router
  // statistics, in LDS that no tile uses any more
  if (fp.stats && ticket == ntot) stats_reduce(fp.st, smem);
}

// ---- backward: weight gradients ------------------------------------------------------

// Per-expert weight gradients: tile (e, mt, nt) of GEMM g sums, over expert
// e's rows r of the permuted order (K, in order, 64 at a time; rows past the
// expert's end read as zero), A[r][mt cols] x B[r][nt cols], both operands
// K-outer (KN), and stores the e-th [M, Nout] block of C. The tiles of one
// expert run together in groups of six row tiles, the row tile fastest, so
// consecutive tiles share a column tile's B panel and a group's A panels are
// re-read from cache (groups of six against four: C2 training step -1.7%,
// C3 -1.6%; two: +0.4%; twelve: -1.4%). BGATHER: B's row r is row row_token[r] of x.
// With a second gradient (C2), an expert's m-tiles are the first gradient's
// then the second's, and all of them share the expert's B panels.
template <bool BGATHER>
__global__ __launch_bounds__(512) void k_gemm_wgrad(WgradParams wp) {
  // the operand stages, then the gather's map ring ([2][64] int32)
  __shared__ __attribute__((aligned(16))) uint16_t smem[dma_lds_elems<256, 256, 2, 64>() + 2 * 64 * 2];
  constexpr int GM = 6;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  GemmParams p = wp.g;
  const int M = wp.M;
  const int mt1 = (M + 255) / 256, ntn = (p.Nout + 255) / 256;
  const int mtn = wp.C2 ? 2 * mt1 : mt1;
  const int per_e = mtn * ntn;
  const int e = L / per_e;
  if (e >= p.N) return;
  const int q = L - e * per_e;
  const int g = q / (GM * ntn);
  const int gm = min(GM, mtn - g * GM);
  const int rq = q - g * GM * ntn;
  TilePos tp{};
  int mt = g * GM + rq % gm;
  if (mt >= mt1) {  // a tile of the second gradient
    mt -= mt1;
    p.A = static_cast<const uint16_t*>(p.A) + wp.a2_col;
    p.C = wp.C2;
  }
  tp.nt = __builtin_amdgcn_readfirstlane(rq / gm);
  tp.ti.expert = 0;
  tp.ti.row0 = __builtin_amdgcn_readfirstlane(mt * 256);
  tp.ti.rows = __builtin_amdgcn_readfirstlane(min(256, M - mt * 256));
  tp.split = __builtin_amdgcn_readfirstlane(e);
  int off = 0, cnt = 0;
  expert_segment(p.offsets, e, static_cast<int>(p.rows_max), off, cnt, p.dbg);
  tp.kb0 = __builtin_amdgcn_readfirstlane(off);
  tp.kb1 = __builtin_amdgcn_readfirstlane(off + cnt);
  tp.KT = (cnt + 63) / 64;
  gemm_tile<256, 256, 4, 2, 2, 64, false, false, NoHook, NoReserve, 2, BGATHER>(p, tp, smem);
}

// ---- launches --------------------------------------------------------------------

int64_t grid_blocks(const GemmParams& p, int BM, int BN) {
  const int NO = p.swiglu ? BN / 2 : BN;
  const int64_t ntiles = (p.Nout + NO - 1) / NO;
  const int64_t mtiles = (p.rows_max + BM - 1) / BM + p.N;
  return ntiles * mtiles * p.splits;
}

template <int BM, int BK, int STAGES, int NW>
hipError_t launch_decode(const GemmParams& p, hipStream_t s) {
  const int64_t blocks = grid_blocks(p, BM, kDecBN);
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), block(NW * 64);
  if (p.swiglu) {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_decode<BM, BK, STAGES, NW, true, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_decode<BM, BK, STAGES, NW, true, false>), grid, block, 0, s, p);
  } else {
    if (p.row_token) hipLaunchKernelGGL((k_gemm_decode<BM, BK, STAGES, NW, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_gemm_decode<BM, BK, STAGES, NW, false, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_bf16_mfma_supported(int K, int Nout) { return K % 8 == 0 && K > 0 && Nout > 0; }

// Experts with few rows on average (decode shapes) take the decode tile in two
// launches; the others the persistent kernel's 256 x 256 tiles.
bool gemm_decode_shape(int64_t rows_max, int N) { return rows_max / (N > 0 ? N : 1) <= 48; }

void gemm_decode_tile(int* bm, int* bn) {
  *bm = kDecBM;
  *bn = kDecBN;
}

int fused_error_index() { return kSchedError; }

int fused_sched_ints(int64_t rows_max, int N) {
  return kSchedDone + static_cast<int>((rows_max + kFusedBM - 1) / kFusedBM) + N + 1;
}

bool gemm_fused_supported(int64_t rows_max, int N, int K1, int F) {
  return !gemm_decode_shape(rows_max, N) && gemm_bf16_mfma_supported(K1, F);
}

hipError_t launch_experts_fused(const FusedParams& fp, hipStream_t s) {
  if (fp.g1.rows_max <= 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // one resident workgroup per compute unit (the LDS stages fill most of a CU)
  const dim3 grid(static_cast<unsigned>(cus > 0 ? cus : 256)), block(4 * 2 * 64);
  if (fp.g1.row_token)
    hipLaunchKernelGGL((k_experts_fused<kFusedBM, kFusedBN, 4, 2, 2, 64, true, true>), grid, block, 0, s, fp);
  else
    hipLaunchKernelGGL((k_experts_fused<kFusedBM, kFusedBN, 4, 2, 2, 64, false, true>), grid, block, 0, s, fp);
  return hipGetLastError();
}

hipError_t launch_bwd_dgrad_fused(const FusedParams& fp, hipStream_t s) {
  if (fp.g1.rows_max <= 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(cus > 0 ? cus : 256)), block(4 * 2 * 64);
  hipLaunchKernelGGL((k_experts_fused<kFusedBM, kFusedBN, 4, 2, 2, 64, false, false>), grid, block, 0, s, fp);
  return hipGetLastError();
}

hipError_t launch_gemm_decode(const GemmParams& p, hipStream_t s) { return launch_decode<kDecBM, 128, 3, 4>(p, s); }

hipError_t launch_gemm_wgrad(const WgradParams& wp, hipStream_t s) {
  const int64_t blocks =
      static_cast<int64_t>((wp.M + 255) / 256) * (wp.C2 ? 2 : 1) * ((wp.g.Nout + 255) / 256) * wp.g.N;
  if (blocks <= 0) return hipSuccess;
  if (wp.g.row_token)
    hipLaunchKernelGGL(k_gemm_wgrad<true>, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, wp);
  else
    hipLaunchKernelGGL(k_gemm_wgrad<false>, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, wp);
  return hipGetLastError();
}

}  // namespace moe
