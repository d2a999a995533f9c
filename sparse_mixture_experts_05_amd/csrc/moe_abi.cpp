// C ABI of the MoE layer: host-side validation, workspace layout and the
// launch sequence of each entry point (declared and documented in moe.h).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "abi_internal.h"
#include "kernels.h"
#include "moe.h"

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// ---- kernel timing -----------------------------------------------------------
// moe_profile_select creates a pool of event pairs once; a timed launch
// records into the next free pair, so the timed region pays two
// hipEventRecord calls per launch and no event creation.
std::mutex g_prof_mu;
int g_prof_kernel = -1;
constexpr size_t kProfPairs = 4096;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_pool;
size_t g_prof_used = 0;

class ProfScope {
 public:
  ProfScope(int kernel, hipStream_t s) : s_(s) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (kernel != g_prof_kernel || g_prof_used >= g_prof_pool.size()) return;
    pair_ = g_prof_pool[g_prof_used++];
    on_ = hipEventRecord(pair_.first, s_) == hipSuccess;
  }
  ~ProfScope() {
    if (on_) (void)hipEventRecord(pair_.second, s_);
  }

 private:
  hipStream_t s_;
  std::pair<hipEvent_t, hipEvent_t> pair_{nullptr, nullptr};
  bool on_ = false;
};

#define MOE_LAUNCH(KID, STREAM, CALL)                                                   \
  do {                                                                                  \
    hipError_t e_;                                                                      \
    {                                                                                   \
      ProfScope ps_(KID, STREAM);                                                       \
      e_ = (CALL);                                                                      \
    }                                                                                   \
    if (e_ != hipSuccess)                                                               \
      return fail(MOE_ERR_DEVICE, "%s launch failed: %s", #KID, hipGetErrorString(e_)); \
  } while (0)

// ---- the expert kernel's bounded wait (test hook) -----------------------------
std::mutex g_wait_mu;
int g_wait_spin = 0;   // <= 0: the default limit
int g_wait_extra = 0;

// ---- configuration -----------------------------------------------------------
constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t A_max = 0;     // upper bound on kept rows
  int hist_tokens = 0;
  int hist_blocks = 0;
  int splits = 1;        // K splits of the down projection in moe_forward
  bool mfma = false;
  bool fused = false;    // both expert GEMMs in one persistent launch
  size_t hist = 0, stat = 0, h = 0, yperm = 0, idx = 0, w = 0, slot = 0, rowtok = 0, counts = 0, kept = 0,
         offsets = 0, sched = 0, dbg = 0, rpart = 0, total = 0;
};

bool use_mfma(const moe_cfg* c) { return c->act == MOE_BF16 && c->F % 8 == 0; }

Layout layout(const moe_cfg* c) {
  Layout L;
  const int64_t T = c->T, Tk = c->T * c->k;
  L.A_max = c->capacity < 0 ? Tk : std::min<int64_t>(Tk, static_cast<int64_t>(c->N) * c->capacity);
  L.hist_tokens = moe::router_tokens_per_block(c->N, c->noisy, c->act == MOE_BF16);
  L.hist_blocks = static_cast<int>((T + L.hist_tokens - 1) / L.hist_tokens);
  L.mfma = use_mfma(c);
  L.fused = L.mfma && moe::gemm_fused_supported(L.A_max, c->N, c->H, c->F);
  if (L.mfma && !L.fused) {
    // decode-shaped tiles: the down projection splits K when there are too
    // few output tiles to spread evenly over 256 compute units (the grid
    // bound below counts a partial row tile per expert, so it overstates the
    // real tiles)
    int bm, bn;
    moe::gemm_decode_tile(&bm, &bn);
    const int64_t tiles = ((L.A_max + bm - 1) / bm + std::min<int64_t>(c->N, L.A_max)) * ((c->H + bn - 1) / bn);
    if (tiles > 0 && tiles < 2048) {
      int64_t s = (2048 + tiles - 1) / tiles;
      s = std::min<int64_t>(s, 8);
      s = std::min<int64_t>(s, std::max<int64_t>(1, c->F / 512));
      L.splits = static_cast<int>(std::max<int64_t>(1, s));
    }
  }
  const size_t act = c->act == MOE_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up(bytes);
    return at;
  };
  L.hist = take(static_cast<size_t>(L.hist_blocks) * c->N * 4);
  L.stat = take(static_cast<size_t>(L.hist_blocks) * c->N * moe::kStatsPerExpert * 4);
  L.h = take(static_cast<size_t>(L.A_max) * c->F * act);
  L.yperm = take(static_cast<size_t>(L.splits) * L.A_max * c->H * 4);
  L.idx = take(static_cast<size_t>(Tk) * 4);
  L.w = take(static_cast<size_t>(Tk) * 4);
  L.slot = take(static_cast<size_t>(Tk) * 4);
  L.rowtok = take(static_cast<size_t>(Tk) * 4);
  L.counts = take(static_cast<size_t>(c->N) * 4);
  L.kept = take(static_cast<size_t>(c->N) * 4);
  L.offsets = take(static_cast<size_t>(c->N + 1) * 4);
  L.sched = take(L.fused ? static_cast<size_t>(moe::fused_sched_ints(L.A_max, c->N)) * 4 : 0);
  L.dbg = take(4);  // the debug word (written by debug builds only)
  L.rpart = take(c->act == MOE_BF16 ? static_cast<size_t>(moe::router_part_floats(T, c->H, c->N, c->noisy)) * 4 : 0);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_ws(const moe_cfg* c, const void* ws, size_t ws_bytes) {
  const size_t need = layout(c).total;
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  if (need > 0 && !ws) return fail(MOE_ERR_INVALID, "workspace pointer is NULL");
  if (ws && !aligned(ws, 256)) return fail(MOE_ERR_INVALID, "workspace must be 256-byte aligned");
  return MOE_OK;
}

#define MOE_REQUIRE(COND, ...)                                 \
  do {                                                         \
    if (!(COND)) return fail(MOE_ERR_INVALID, __VA_ARGS__);    \
  } while (0)

moe_status zero_expert_outputs(const moe_cfg* c, int32_t* a, int32_t* b, int32_t* offsets, float* f0, float* f1,
                               float* bal, hipStream_t s) {
  const int N = c->N;
  hipError_t e = hipSuccess;
  if (a && e == hipSuccess) e = moe::launch_fill_i32(a, N, 0, s);
  if (b && e == hipSuccess) e = moe::launch_fill_i32(b, N, 0, s);
  if (offsets && e == hipSuccess) e = moe::launch_fill_i32(offsets, N + 1, 0, s);
  if (f0 && e == hipSuccess) e = moe::launch_fill_f32(f0, N, 0.0f, s);
  if (f1 && e == hipSuccess) e = moe::launch_fill_f32(f1, N, 0.0f, s);
  if (bal && e == hipSuccess) e = moe::launch_fill_f32(bal, 1, 0.0f, s);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "fill launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

// sched_zeroed: the fused kernel's queue counters were already zeroed on the
// stream (by the scatter in moe_forward). stats_tail: router statistics for
// the fused kernel to reduce once its queue is empty (only when L.fused).
moe_status run_gemms(const moe_cfg* c, const Layout& L, const void* a, const int32_t* row_token,
                     const int32_t* offsets, const void* Wgate, const void* Wup, const void* Wdown, float* y_perm,
                     int splits, void* ws, bool sched_zeroed, hipStream_t s,
                     const moe::StatsParams* stats_tail = nullptr, float* gu = nullptr, int32_t* dbg = nullptr) {
  const int bf16 = c->act == MOE_BF16;
  moe::GemmParams g1{};
  g1.A = a;
  g1.lda = c->H;
  g1.row_token = row_token;
  g1.offsets = offsets;
  g1.N = c->N;
  g1.B0 = Wgate;
  g1.B1 = Wup;
  g1.b_expert_stride = static_cast<int64_t>(c->F) * c->H;
  g1.ldb = c->H;
  g1.K = c->H;
  g1.Nout = c->F;
  g1.C = at<char>(ws, L.h);
  g1.ldc = c->F;
  g1.c_split_stride = 0;
  g1.splits = 1;
  g1.rows_max = L.A_max;
  g1.a_rows = row_token ? c->T : c->T * c->k;
  g1.swiglu = 1;
  g1.gu = gu;
  g1.dbg = dbg ? dbg : at<int32_t>(ws, L.dbg);
  moe::GemmParams g2 = g1;
  g2.gu = nullptr;
  g2.A = at<char>(ws, L.h);
  g2.lda = c->F;
  g2.row_token = nullptr;
  g2.B0 = Wdown;
  g2.B1 = nullptr;
  g2.b_expert_stride = static_cast<int64_t>(c->H) * c->F;
  g2.ldb = c->F;
  g2.K = c->F;
  g2.Nout = c->H;
  g2.C = y_perm;
  g2.ldc = c->H;
  g2.c_split_stride = L.A_max * static_cast<int64_t>(c->H);
  g2.a_rows = L.A_max;
  g2.splits = splits;
  g2.swiglu = 0;
  if (L.fused) {
    g2.splits = 1;
    int32_t* sched = at<int32_t>(ws, L.sched);
    if (!sched_zeroed) {
      hipError_t e = moe::launch_fill_i32(sched, moe::fused_sched_ints(L.A_max, c->N), 0, s);
      if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "fill launch failed: %s", hipGetErrorString(e));
    }
    int spin = moe::kDefaultSpinLimit, extra = 0;
    {
      std::lock_guard<std::mutex> lk(g_wait_mu);
      if (g_wait_spin > 0) spin = g_wait_spin;
      extra = g_wait_extra;
    }
    moe::FusedParams fp{g1, g2, sched, stats_tail ? *stats_tail : moe::StatsParams{}, stats_tail ? 1 : 0, spin, extra};
    MOE_LAUNCH(MOE_KERNEL_EXPERTS, s, moe::launch_experts_fused(fp, s));
  } else if (L.mfma) {
    MOE_LAUNCH(MOE_KERNEL_GEMM1, s, moe::launch_gemm_decode(g1, s));
    MOE_LAUNCH(MOE_KERNEL_GEMM2, s, moe::launch_gemm_decode(g2, s));
  } else {
    MOE_LAUNCH(MOE_KERNEL_GEMM1, s, moe::launch_gemm_simple(g1, bf16, s));
    MOE_LAUNCH(MOE_KERNEL_GEMM2, s, moe::launch_gemm_simple(g2, bf16, s));
  }
  return MOE_OK;
}

// The routed layer's launches after validation: router (and statistics),
// scatter, expert GEMMs and combine. res: the residual layer's shared-slice
// output, added by the combine, or null.
struct Residual {
  const float* y;        // [splits][T][H] fp32 partial sums
  int64_t split_stride;  // elements
  int splits;
};

// What a training forward keeps for the backward (in the training workspace).
struct TrainSave {
  float* logits;         // [T,N] clean logits
  float* noise_logits;   // [T,N] (noisy)
  float* gu;             // [A_max, 2F] g and u
};

moe_status forward_launch(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                          const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* topk_idx_opt,
                          float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt, float* importance_opt,
                          float* P_opt, float* balance_opt, float* smooth_load_opt, bool stats, void* ws,
                          const Residual* res, hipStream_t s, const TrainSave* train = nullptr) {
  const Layout L = layout(c);
  int32_t* topk_idx = topk_idx_opt ? topk_idx_opt : at<int32_t>(ws, L.idx);
  float* topk_w = topk_w_opt ? topk_w_opt : at<float>(ws, L.w);
  int32_t* slot = at<int32_t>(ws, L.slot);
  int32_t* row_token = at<int32_t>(ws, L.rowtok);
  int32_t* offsets = at<int32_t>(ws, L.offsets);

  moe::RouterParams rp{};
  rp.x = x;
  rp.act_bf16 = c->act == MOE_BF16;
  rp.Wg = Wg;
  rp.Wn = Wn;
  rp.eps = eps;
  rp.T = c->T;
  rp.H = c->H;
  rp.N = c->N;
  rp.k = c->k;
  rp.order = c->order;
  rp.noisy = c->noisy;
  rp.logits = train ? train->logits : nullptr;
  rp.noise_logits = train ? train->noise_logits : nullptr;
  rp.topk_idx = topk_idx;
  rp.topk_w = topk_w;
  rp.hist = at<int32_t>(ws, L.hist);
  rp.stat_part = stats ? at<float>(ws, L.stat) : nullptr;
  rp.smooth = stats && smooth_load_opt ? 1 : 0;
  rp.part = at<float>(ws, L.rpart);
  MOE_LAUNCH(MOE_KERNEL_ROUTER, s, moe::launch_router(rp, s));
  // statistics: reduced by the persistent expert kernel once its queue is
  // empty when that kernel runs, else by a launch of their own
  const moe::StatsParams sp{at<int32_t>(ws, L.hist), at<float>(ws, L.stat), L.hist_blocks, c->T, c->N, c->k,
                            load_opt, importance_opt, P_opt, balance_opt, smooth_load_opt};
  if (stats && !L.fused) MOE_LAUNCH(MOE_KERNEL_STATS, s, moe::launch_stats(sp, s));
  moe::ScatterParams sc{topk_idx, at<int32_t>(ws, L.hist), L.hist_tokens, c->T, c->N, c->k, c->capacity,
                        (!stats && load_opt && !train) ? load_opt : at<int32_t>(ws, L.counts), kept_opt, offsets, slot,
                        row_token, L.fused ? at<int32_t>(ws, L.sched) : nullptr,
                        L.fused ? moe::fused_sched_ints(L.A_max, c->N) : 0, at<int32_t>(ws, L.dbg)};
  MOE_LAUNCH(MOE_KERNEL_SCATTER, s, moe::launch_scatter(sc, s));
  if (train && !stats && load_opt) {
    const hipError_t e = hipMemcpyAsync(load_opt, at<int32_t>(ws, L.counts), sizeof(int32_t) * c->N,
                                        hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "copy of the expert counts failed: %s", hipGetErrorString(e));
  }
  float* y_perm = at<float>(ws, L.yperm);
  const moe_status st = run_gemms(c, L, x, row_token, offsets, Wgate, Wup, Wdown, y_perm, L.splits, ws, true, s,
                                  stats && L.fused ? &sp : nullptr, train ? train->gu : nullptr);
  if (st != MOE_OK) return st;
  moe::CombineParams cp{y_perm, L.A_max * static_cast<int64_t>(c->H), L.splits, slot, topk_w, y,
                        c->out == MOE_BF16, c->T, c->H, c->k, c->out_scale,
                        L.fused ? at<int32_t>(ws, L.sched) + moe::fused_error_index() : nullptr,
                        res ? res->y : nullptr, res ? res->split_stride : 0, res ? res->splits : 0, L.A_max,
                        at<int32_t>(ws, L.dbg)};
  MOE_LAUNCH(MOE_KERNEL_COMBINE, s, moe::launch_combine(cp, s));
  return MOE_OK;
}

}  // namespace

namespace moe {

moe_status set_error(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace moe

extern "C" {

int32_t moe_capacity(int64_t T, int32_t N, int32_t k, double cf, int32_t count_assignments) {
  if (cf < 0 || N <= 0 || T < 0 || k <= 0 || !std::isfinite(cf)) return -1;
  const double num = count_assignments ? static_cast<double>(T) * k : static_cast<double>(T);
  const double c = std::ceil(cf * num / N - 1e-9);
  if (c > 2147483647.0) return -1;
  return static_cast<int32_t>(c < 0 ? 0 : c);
}

moe_status moe_check(const moe_cfg* c) {
  g_err.clear();
  if (!c) return fail(MOE_ERR_INVALID, "cfg is NULL");
  if (c->T < 0) return fail(MOE_ERR_INVALID, "T = %lld < 0", static_cast<long long>(c->T));
  if (c->T > (int64_t(1) << 26)) return fail(MOE_ERR_UNSUPPORTED, "T above 2^26");
  if (c->H < 1 || c->F < 1) return fail(MOE_ERR_INVALID, "H and F must be >= 1");
  if (c->N < 1 || c->k < 1 || c->k > c->N) return fail(MOE_ERR_INVALID, "need 1 <= k <= N (N=%d, k=%d)", c->N, c->k);
  if (c->N > 64) return fail(MOE_ERR_UNSUPPORTED, "N = %d above 64", c->N);
  if (c->H % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "H = %d is not a multiple of 8", c->H);
  if (c->order != MOE_TOPK_THEN_SOFTMAX && c->order != MOE_SOFTMAX_THEN_TOPK)
    return fail(MOE_ERR_INVALID, "unknown order %d", c->order);
  if ((c->noisy != 0 && c->noisy != 1) || (c->want_stats != 0 && c->want_stats != 1))
    return fail(MOE_ERR_INVALID, "noisy and want_stats must be 0 or 1");
  if (!std::isfinite(c->out_scale)) return fail(MOE_ERR_INVALID, "out_scale is not finite");
  const bool dt_ok = (c->act == MOE_BF16 || c->act == MOE_F32) && (c->wt == MOE_BF16 || c->wt == MOE_F32) &&
                     (c->out == MOE_BF16 || c->out == MOE_F32);
  if (!dt_ok) return fail(MOE_ERR_INVALID, "unknown dtype code");
  if (c->act != c->wt) return fail(MOE_ERR_UNSUPPORTED, "activations and expert weights must share a dtype");
  // the kernels address each operand with 32-bit byte offsets below 2^31
  const int64_t Tk = c->T * c->k;
  const int64_t lim = int64_t(1) << 29;  // elements, so that fp32 operands stay below 2 GiB
  if (c->T * static_cast<int64_t>(c->H) >= lim || Tk * static_cast<int64_t>(c->F) >= lim ||
      Tk * static_cast<int64_t>(c->H) >= lim || static_cast<int64_t>(c->F) * c->H >= lim)
    return fail(MOE_ERR_UNSUPPORTED, "T*H, T*k*F, T*k*H and F*H must stay below 2^29 elements");
  // the matrix-core router's partial logits (one T x N(1 + noisy) set per
  // chunk of H) and the noise draws are addressed the same way
  if (c->act == MOE_BF16 && moe::router_part_floats(c->T, c->H, c->N, c->noisy) >= lim)
    return fail(MOE_ERR_UNSUPPORTED, "the router's partial logits (T*N*(1+noisy) per chunk of H) must stay below "
                                     "2^29 floats");
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_cfg* c) {
  if (moe_check(c) != MOE_OK) return 0;
  return layout(c).total;
}

moe_status moe_route(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                     float* logits_opt, int32_t* topk_idx, float* topk_w, int32_t* load_opt,
                     float* importance_opt, float* P_opt, float* balance_opt, float* smooth_load_opt, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(!smooth_load_opt || c->noisy, "the smooth load needs the noisy gate (cfg->noisy = 1)");
  const bool stats = c->want_stats && (load_opt || importance_opt || P_opt || balance_opt || smooth_load_opt);
  if (c->T == 0) {
    if (stats) {
      st = zero_expert_outputs(c, load_opt, nullptr, nullptr, importance_opt, P_opt, balance_opt, s);
      if (st == MOE_OK && smooth_load_opt) st = zero_expert_outputs(c, nullptr, nullptr, nullptr, smooth_load_opt,
                                                                     nullptr, nullptr, s);
      return st;
    }
    return MOE_OK;
  }
  MOE_REQUIRE(x && Wg && topk_idx && topk_w, "x, Wg, topk_idx and topk_w are required");
  MOE_REQUIRE(!c->noisy || (Wn && eps), "noisy routing needs Wn and eps");
  MOE_REQUIRE(aligned(x, 16) && aligned(Wg, 16) && (!Wn || aligned(Wn, 16)), "x, Wg and Wn must be 16-byte aligned");
  // the workspace holds the statistics' partials and the matrix-core
  // router's partial logits
  const bool need_ws = stats || c->act == MOE_BF16;
  if (need_ws) {
    st = check_ws(c, ws, ws_bytes);
    if (st != MOE_OK) return st;
  }
  const Layout L = layout(c);
  moe::RouterParams rp{};
  rp.x = x;
  rp.act_bf16 = c->act == MOE_BF16;
  rp.Wg = Wg;
  rp.Wn = Wn;
  rp.eps = eps;
  rp.T = c->T;
  rp.H = c->H;
  rp.N = c->N;
  rp.k = c->k;
  rp.order = c->order;
  rp.noisy = c->noisy;
  rp.logits = logits_opt;
  rp.topk_idx = topk_idx;
  rp.topk_w = topk_w;
  rp.hist = stats ? at<int32_t>(ws, L.hist) : nullptr;
  rp.stat_part = stats ? at<float>(ws, L.stat) : nullptr;
  rp.smooth = stats && smooth_load_opt ? 1 : 0;
  rp.part = c->act == MOE_BF16 ? at<float>(ws, L.rpart) : nullptr;
  MOE_LAUNCH(MOE_KERNEL_ROUTER, s, moe::launch_router(rp, s));
  if (stats) {
    moe::StatsParams sp{at<int32_t>(ws, L.hist), at<float>(ws, L.stat), L.hist_blocks, c->T, c->N, c->k,
                        load_opt, importance_opt, P_opt, balance_opt, smooth_load_opt};
    MOE_LAUNCH(MOE_KERNEL_STATS, s, moe::launch_stats(sp, s));
  }
  return MOE_OK;
}

moe_status moe_permute(const moe_cfg* c, const void* x, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* row_token, void* x_perm, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(counts && offsets, "counts and offsets are required");
  if (c->T == 0) return zero_expert_outputs(c, counts, nullptr, offsets, nullptr, nullptr, nullptr, s);
  MOE_REQUIRE(topk_idx && slot && row_token, "topk_idx, slot and row_token are required");
  MOE_REQUIRE(!x_perm || (x && aligned(x, 16) && aligned(x_perm, 16)), "gather needs 16-byte aligned x and x_perm");
  st = check_ws(c, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const Layout L = layout(c);
  moe::HistParams hp{topk_idx, c->T, c->N, c->k, L.hist_tokens, at<int32_t>(ws, L.hist)};
  MOE_LAUNCH(MOE_KERNEL_HIST, s, moe::launch_hist(hp, s));
  moe::ScatterParams sp{topk_idx, at<int32_t>(ws, L.hist), L.hist_tokens, c->T, c->N, c->k, c->capacity,
                        counts, nullptr, offsets, slot, row_token, nullptr, 0, at<int32_t>(ws, L.dbg)};
  MOE_LAUNCH(MOE_KERNEL_SCATTER, s, moe::launch_scatter(sp, s));
  if (x_perm) {
    moe::GatherParams gp{x,   x_perm, row_token, offsets, c->T * c->k, c->H, c->N, c->act == MOE_BF16 ? 2 : 4,
                         c->T, at<int32_t>(ws, L.dbg)};
    MOE_LAUNCH(MOE_KERNEL_GATHER, s, moe::launch_gather(gp, s));
  }
  return MOE_OK;
}

moe_status moe_grouped_swiglu(const moe_cfg* c, const void* a, const int32_t* row_token_opt,
                              const int32_t* offsets, const void* Wgate, const void* Wup, const void* Wdown,
                              float* y_perm, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  if (c->T == 0) return MOE_OK;
  MOE_REQUIRE(a && offsets && Wgate && Wup && Wdown && y_perm, "inputs and y_perm are required");
  MOE_REQUIRE(aligned(a, 16) && aligned(Wgate, 16) && aligned(Wup, 16) && aligned(Wdown, 16) && aligned(y_perm, 16),
              "activations, weights and y_perm must be 16-byte aligned");
  st = check_ws(c, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const Layout L = layout(c);
  return run_gemms(c, L, a, row_token_opt, offsets, Wgate, Wup, Wdown, y_perm, 1, ws, false, s);
}

moe_status moe_combine(const moe_cfg* c, const float* y_perm, const int32_t* slot, const float* topk_w, void* y,
                       hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  if (c->T == 0) return MOE_OK;
  MOE_REQUIRE(y_perm && slot && topk_w && y, "y_perm, slot, topk_w and y are required");
  MOE_REQUIRE(aligned(y_perm, 16) && aligned(y, 16), "y_perm and y must be 16-byte aligned");
  moe::CombineParams cp{y_perm, 0, 1, slot, topk_w, y, c->out == MOE_BF16, c->T, c->H, c->k, c->out_scale,
                        nullptr, nullptr, 0, 0, c->T * c->k, nullptr};
  MOE_LAUNCH(MOE_KERNEL_COMBINE, s, moe::launch_combine(cp, s));
  return MOE_OK;
}

moe_status moe_forward(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                       const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* topk_idx_opt,
                       float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt, float* importance_opt,
                       float* P_opt, float* balance_opt, float* smooth_load_opt, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(!smooth_load_opt || c->noisy, "the smooth load needs the noisy gate (cfg->noisy = 1)");
  const bool stats = c->want_stats && (load_opt || importance_opt || P_opt || balance_opt || smooth_load_opt);
  if (c->T == 0) {
    st = zero_expert_outputs(c, kept_opt, load_opt, nullptr, stats ? importance_opt : nullptr,
                             stats ? P_opt : nullptr, stats ? balance_opt : nullptr, s);
    if (st == MOE_OK && stats && smooth_load_opt)
      st = zero_expert_outputs(c, nullptr, nullptr, nullptr, smooth_load_opt, nullptr, nullptr, s);
    return st;
  }
  MOE_REQUIRE(x && Wg && Wgate && Wup && Wdown && y, "x, Wg, expert weights and y are required");
  MOE_REQUIRE(!c->noisy || (Wn && eps), "noisy routing needs Wn and eps");
  MOE_REQUIRE(aligned(x, 16) && aligned(Wg, 16) && (!Wn || aligned(Wn, 16)) && aligned(Wgate, 16) &&
                  aligned(Wup, 16) && aligned(Wdown, 16) && aligned(y, 16),
              "x, router and expert weights and y must be 16-byte aligned");
  st = check_ws(c, ws, ws_bytes);
  if (st != MOE_OK) return st;
  return forward_launch(c, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, topk_idx_opt, topk_w_opt, kept_opt, load_opt,
                        importance_opt, P_opt, balance_opt, smooth_load_opt, stats, ws, nullptr, s);
}

// The residual layer's shared slice: a one-expert layer over all T rows
// (gate/up width F_shared), whose workspace follows the routed layer's.
static moe_cfg shared_cfg(const moe_cfg* c, int32_t F_shared) {
  moe_cfg sc = *c;
  sc.F = F_shared;
  sc.N = 1;
  sc.k = 1;
  sc.capacity = -1;
  sc.order = MOE_TOPK_THEN_SOFTMAX;
  sc.noisy = 0;
  sc.want_stats = 0;
  sc.out_scale = 1.0f;
  return sc;
}

size_t moe_residual_workspace_bytes(const moe_cfg* c, int32_t F_shared) {
  if (moe_check(c) != MOE_OK || F_shared < 1) return 0;
  const moe_cfg sc = shared_cfg(c, F_shared);
  if (moe_check(&sc) != MOE_OK) return 0;
  return layout(c).total + layout(&sc).total;
}

moe_status moe_forward_residual(const moe_cfg* c, int32_t F_shared, const void* x, const float* Wg, const float* Wn,
                                const float* eps, const void* Wgate, const void* Wup, const void* Wdown,
                                const void* Ws_gate, const void* Ws_up, const void* Ws_down, void* y,
                                int32_t* topk_idx_opt, float* topk_w_opt, int32_t* kept_opt, int32_t* load_opt,
                                float* importance_opt, float* P_opt, float* balance_opt, float* smooth_load_opt,
                                void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(F_shared >= 1, "F_shared = %d: the shared slice needs at least one neuron", F_shared);
  const moe_cfg sc = shared_cfg(c, F_shared);
  st = moe_check(&sc);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(!smooth_load_opt || c->noisy, "the smooth load needs the noisy gate (cfg->noisy = 1)");
  const bool stats = c->want_stats && (load_opt || importance_opt || P_opt || balance_opt || smooth_load_opt);
  if (c->T == 0) {
    st = zero_expert_outputs(c, kept_opt, load_opt, nullptr, stats ? importance_opt : nullptr,
                             stats ? P_opt : nullptr, stats ? balance_opt : nullptr, s);
    if (st == MOE_OK && stats && smooth_load_opt)
      st = zero_expert_outputs(c, nullptr, nullptr, nullptr, smooth_load_opt, nullptr, nullptr, s);
    return st;
  }
  MOE_REQUIRE(x && Wg && Wgate && Wup && Wdown && Ws_gate && Ws_up && Ws_down && y,
              "x, Wg, expert and shared-slice weights and y are required");
  MOE_REQUIRE(!c->noisy || (Wn && eps), "noisy routing needs Wn and eps");
  MOE_REQUIRE(aligned(x, 16) && aligned(Wg, 16) && (!Wn || aligned(Wn, 16)) && aligned(Wgate, 16) &&
                  aligned(Wup, 16) && aligned(Wdown, 16) && aligned(Ws_gate, 16) && aligned(Ws_up, 16) &&
                  aligned(Ws_down, 16) && aligned(y, 16),
              "x, router, expert and shared-slice weights and y must be 16-byte aligned");
  const size_t need = moe_residual_workspace_bytes(c, F_shared);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  MOE_REQUIRE(ws && aligned(ws, 256), "the workspace must be non-NULL and 256-byte aligned");
  // the shared slice first (it does not depend on the routing): rows 0..T-1
  // of its one expert are the tokens themselves
  const Layout L = layout(c), Ls = layout(&sc);
  void* ws_s = static_cast<char*>(ws) + L.total;
  int32_t* offsets_s = at<int32_t>(ws_s, Ls.offsets);
  hipError_t e = moe::launch_fill_i32(offsets_s, 1, 0, s);
  if (e == hipSuccess) e = moe::launch_fill_i32(offsets_s + 1, 1, static_cast<int32_t>(c->T), s);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "fill launch failed: %s", hipGetErrorString(e));
  float* y_s = at<float>(ws_s, Ls.yperm);
  st = run_gemms(&sc, Ls, x, nullptr, offsets_s, Ws_gate, Ws_up, Ws_down, y_s, Ls.splits, ws_s, false, s, nullptr,
                 nullptr, at<int32_t>(ws, L.dbg));
  if (st != MOE_OK) return st;
  const Residual res{y_s, Ls.A_max * static_cast<int64_t>(c->H), Ls.splits};
  return forward_launch(c, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, topk_idx_opt, topk_w_opt, kept_opt, load_opt,
                        importance_opt, P_opt, balance_opt, smooth_load_opt, stats, ws, &res, s);
}

}  // extern "C"

// ---- training: forward that keeps what the backward needs, and the backward ----
namespace {

// The training workspace: the forward's layout, then what the training
// forward keeps (router logits, g and u) and the backward's buffers.
struct TrainLayout {
  Layout L;
  size_t logits = 0, nlog = 0, gu = 0, dE = 0, dgu = 0, dxp = 0, dlog = 0, dnz = 0, rwp = 0, total = 0;
};

TrainLayout train_layout(const moe_cfg* c) {
  TrainLayout t;
  t.L = layout(c);
  const int64_t T = c->T, H = c->H, F = c->F, N = c->N, A = t.L.A_max;
  size_t o = t.L.total;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o += up(bytes);
    return at_;
  };
  t.logits = take(T * N * 4);
  t.nlog = take(T * N * 4);
  t.gu = take(A * 2 * F * 4);
  t.dE = take(A * H * 2);
  t.dgu = take(A * 2 * F * 2);
  t.dxp = take(A * H * 4);
  t.dlog = take(T * N * 4);
  t.dnz = take(T * N * 4);
  t.rwp = take(static_cast<size_t>(moe::router_wgrad_chunks(T)) * H * N * 2 * 4);
  t.total = o;
  return t;
}

// The backward runs on the persistent-kernel path only: bf16, F % 8 == 0,
// prefill shapes (more than 48 rows per expert on average).
moe_status check_train(const moe_cfg* c) {
  moe_status st = moe_check(c);
  if (st != MOE_OK) return st;
  const Layout L = layout(c);
  if (!L.fused)
    return fail(MOE_ERR_UNSUPPORTED,
                "training needs bf16 activations and weights, F %% 8 == 0 and more than 48 rows per expert on "
                "average (the persistent expert kernel's shapes)");
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_train_workspace_bytes(const moe_cfg* c) {
  if (check_train(c) != MOE_OK) return 0;
  return train_layout(c).total;
}

moe_status moe_forward_train(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                             const void* Wgate, const void* Wup, const void* Wdown, void* y, int32_t* kept_opt,
                             int32_t* load_opt, float* importance_opt, float* P_opt, float* balance_opt,
                             float* smooth_load_opt, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = check_train(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(!smooth_load_opt || c->noisy, "the smooth load needs the noisy gate (cfg->noisy = 1)");
  const bool stats = c->want_stats && (load_opt || importance_opt || P_opt || balance_opt || smooth_load_opt);
  if (c->T == 0) {
    st = zero_expert_outputs(c, kept_opt, load_opt, nullptr, stats ? importance_opt : nullptr,
                             stats ? P_opt : nullptr, stats ? balance_opt : nullptr, s);
    if (st == MOE_OK && stats && smooth_load_opt)
      st = zero_expert_outputs(c, nullptr, nullptr, nullptr, smooth_load_opt, nullptr, nullptr, s);
    return st;
  }
  MOE_REQUIRE(x && Wg && Wgate && Wup && Wdown && y, "x, Wg, expert weights and y are required");
  MOE_REQUIRE(!c->noisy || (Wn && eps), "noisy routing needs Wn and eps");
  MOE_REQUIRE(aligned(x, 16) && aligned(Wg, 16) && (!Wn || aligned(Wn, 16)) && aligned(Wgate, 16) &&
                  aligned(Wup, 16) && aligned(Wdown, 16) && aligned(y, 16),
              "x, router and expert weights and y must be 16-byte aligned");
  const TrainLayout t = train_layout(c);
  if (ws_bytes < t.total) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, t.total);
  MOE_REQUIRE(ws && aligned(ws, 256), "the workspace must be non-NULL and 256-byte aligned");
  const TrainSave save{at<float>(ws, t.logits), c->noisy ? at<float>(ws, t.nlog) : nullptr, at<float>(ws, t.gu)};
  return forward_launch(c, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, nullptr, nullptr, kept_opt, load_opt,
                        importance_opt, P_opt, balance_opt, smooth_load_opt, stats, ws, nullptr, s, &save);
}

moe_status moe_backward(const moe_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                        const void* Wgate, const void* Wup, const void* Wdown, const float* dy, float d_balance,
                        float* dx, float* dWg, float* dWn_opt, float* dWgate, float* dWup, float* dWdown, void* ws,
                        size_t ws_bytes, hipStream_t s) {
  moe_status st = check_train(c);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(std::isfinite(d_balance), "d_balance is not finite");
  MOE_REQUIRE(dx && dWg && dWgate && dWup && dWdown, "dx and every weight gradient are required");
  MOE_REQUIRE(!c->noisy || dWn_opt, "the noisy gate needs dWn");
  const int64_t T = c->T, H = c->H, F = c->F, N = c->N;
  if (T == 0) {
    hipError_t e = moe::launch_fill_f32(dWg, H * N, 0.0f, s);
    if (e == hipSuccess && dWn_opt) e = moe::launch_fill_f32(dWn_opt, H * N, 0.0f, s);
    if (e == hipSuccess) e = moe::launch_fill_f32(dWgate, N * F * H, 0.0f, s);
    if (e == hipSuccess) e = moe::launch_fill_f32(dWup, N * F * H, 0.0f, s);
    if (e == hipSuccess) e = moe::launch_fill_f32(dWdown, N * H * F, 0.0f, s);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "fill launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
  }
  MOE_REQUIRE(x && Wg && Wgate && Wup && Wdown && dy, "x, Wg, expert weights and dy are required");
  MOE_REQUIRE(!c->noisy || (Wn && eps), "noisy routing needs Wn and eps");
  MOE_REQUIRE(aligned(x, 16) && aligned(Wg, 16) && aligned(Wgate, 16) && aligned(Wup, 16) && aligned(Wdown, 16) &&
                  aligned(dy, 16) && aligned(dx, 16) && aligned(dWgate, 16) && aligned(dWup, 16) &&
                  aligned(dWdown, 16),
              "inputs and gradients must be 16-byte aligned");
  const TrainLayout t = train_layout(c);
  if (ws_bytes < t.total) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, t.total);
  MOE_REQUIRE(ws && aligned(ws, 256), "the workspace must be non-NULL and 256-byte aligned");
  const Layout& L = t.L;
  const int A = static_cast<int>(L.A_max);
  const int32_t* offsets = at<int32_t>(ws, L.offsets);
  uint16_t* dE = at<uint16_t>(ws, t.dE);
  uint16_t* dgu = at<uint16_t>(ws, t.dgu);
  float* dlog = at<float>(ws, t.dlog);
  float* dnz = at<float>(ws, t.dnz);

  // gate weights back to the router; dE = s w dy at every kept slot's row
  moe::BwdGateParams gp{T, c->H, c->N, c->k, c->order, c->noisy, c->out_scale, d_balance, dy,
                        at<float>(ws, L.yperm), at<int32_t>(ws, L.slot), at<int32_t>(ws, L.idx), at<float>(ws, L.w),
                        at<float>(ws, t.logits), c->noisy ? at<float>(ws, t.nlog) : nullptr, eps,
                        at<int32_t>(ws, L.counts), dE, dlog, dnz, L.A_max, at<int32_t>(ws, L.dbg)};
  // its first workgroup also zeroes the queue of the persistent launch below
  int32_t* sched = at<int32_t>(ws, L.sched);
  gp.zero = sched;
  gp.zero_n = moe::fused_sched_ints(L.A_max, c->N);
  MOE_LAUNCH(MOE_KERNEL_BWD_GATE, s, moe::launch_bwd_gate(gp, s));

  // dh = dE . Wdown_e (B = Wdown_e[h][f], K = h, read in place), and the
  // SwiGLU derivative into dg | du (bf16)
  moe::GemmParams gd{};
  gd.A = dE;
  gd.lda = H;
  gd.offsets = offsets;
  gd.N = c->N;
  gd.B0 = Wdown;
  gd.b_expert_stride = H * F;
  gd.ldb = F;
  gd.b_rows = H;
  gd.ksplit = c->H;
  gd.K = c->H;
  gd.Nout = c->F;
  gd.C = dgu;
  gd.ldc = 2 * F;
  gd.splits = 1;
  gd.rows_max = A;
  gd.a_rows = A;
  gd.gu = at<float>(ws, t.gu);
  gd.epi = 1;
  gd.dbg = at<int32_t>(ws, L.dbg);
  // dx_perm = dg . Wgate_e + du . Wup_e: K runs over the 2F columns of dg | du,
  // B row k is Wgate_e row k (k < F) or Wup_e row k - F; in the same
  // persistent launch, each row block's dx tiles after its dh tiles
  moe::GemmParams gx{};
  gx.A = dgu;
  gx.lda = 2 * F;
  gx.offsets = offsets;
  gx.N = c->N;
  gx.B0 = Wgate;
  gx.B1 = Wup;
  gx.b_expert_stride = F * H;
  gx.ldb = H;
  gx.b_rows = F;
  gx.ksplit = c->F;
  gx.K = 2 * c->F;
  gx.Nout = c->H;
  gx.C = at<float>(ws, t.dxp);
  gx.ldc = H;
  gx.splits = 1;
  gx.rows_max = A;
  gx.a_rows = A;
  gx.dbg = gd.dbg;
  // dWdown_e[h][f] = sum over the expert's rows r of dE[r][h] h[r][f], both
  // operands K-outer: it needs nothing from this launch, so its tiles run
  // from the same queue and fill the units the dependent dx tiles leave idle
  moe::WgradParams wd{};
  moe::GemmParams& w0 = wd.g;
  w0.offsets = offsets;
  w0.N = c->N;
  w0.rows_max = A;
  w0.splits = 1;
  w0.A = dE;
  w0.lda = H;
  w0.a_rows = A;
  w0.B0 = at<uint16_t>(ws, L.h);
  w0.ldb = F;
  w0.b_rows = A;
  w0.Nout = c->F;
  w0.C = dWdown;
  w0.ldc = F;
  w0.c_split_stride = H * F;
  w0.dbg = gd.dbg;
  wd.M = c->H;
  {
    int spin = moe::kDefaultSpinLimit, extra = 0;
    {
      std::lock_guard<std::mutex> lk(g_wait_mu);
      if (g_wait_spin > 0) spin = g_wait_spin;
      extra = g_wait_extra;
    }
    const moe::FusedParams fp{gd, gx, sched, moe::StatsParams{}, 0, spin, extra, wd.g, wd.M};
    MOE_LAUNCH(MOE_KERNEL_BWD_DGRAD, s, moe::launch_bwd_dgrad_fused(fp, s));
  }
  // dx = sum of the slots' rows + the router terms
  moe::BwdDxParams dp{T,  c->H, c->N, c->k, c->noisy, at<float>(ws, t.dxp), L.A_max, at<int32_t>(ws, L.slot), dlog,
                      dnz, Wg, Wn, dx, gd.dbg};
  MOE_LAUNCH(MOE_KERNEL_BWD_DX, s, moe::launch_bwd_dx(dp, s));
  // the other weight gradients per expert, K over the expert's rows of the
  // permuted order, both in one launch whose XCD-aware order keeps an
  // expert's tiles (which share its gathered x panels) together
  moe::WgradParams wg = wd;  // dWgate_e[f][h] = sum_r dg[r][f] x[row_token[r]][h]
  wg.g.A = dgu;
  wg.g.lda = 2 * F;
  wg.g.B0 = x;
  wg.g.ldb = H;
  wg.g.b_rows = T;
  wg.g.row_token = at<int32_t>(ws, L.rowtok);
  wg.g.Nout = c->H;
  wg.g.C = dWgate;
  wg.g.ldc = H;
  wg.g.c_split_stride = F * H;
  wg.M = c->F;
  wg.C2 = dWup;  // dWup_e: the du half of dg | du
  wg.a2_col = F;
  MOE_LAUNCH(MOE_KERNEL_BWD_WGRAD, s, moe::launch_gemm_wgrad(wg, s));
  // router weights
  moe::RouterWgradParams rw{T, c->H, c->N, c->noisy, static_cast<const uint16_t*>(x), dlog, dnz,
                            at<float>(ws, t.rwp), dWg, dWn_opt};
  MOE_LAUNCH(MOE_KERNEL_BWD_ROUTER, s, moe::launch_router_wgrad(rw, s));
  return MOE_OK;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "unknown moe_status";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_debug_set_wait(int32_t spin_limit, int32_t wait_extra) {
  if (wait_extra < 0) return fail(MOE_ERR_INVALID, "wait_extra = %d < 0", wait_extra);
  std::lock_guard<std::mutex> lk(g_wait_mu);
  g_wait_spin = spin_limit;
  g_wait_extra = wait_extra;
  return MOE_OK;
}

int32_t moe_debug_build(void) {
#ifdef MOE_DEBUG
  return 1;
#else
  return 0;
#endif
}

size_t moe_debug_word_offset(const moe_cfg* c) {
  if (moe_check(c) != MOE_OK) return 0;
  return layout(c).dbg;
}

moe_status moe_profile_select(int32_t kernel_id) {
  if (kernel_id < -1 || kernel_id >= MOE_KERNEL_COUNT) return fail(MOE_ERR_INVALID, "unknown kernel id %d", kernel_id);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (kernel_id >= 0 && g_prof_pool.empty()) {
    for (size_t i = 0; i < kProfPairs; ++i) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
        return fail(MOE_ERR_DEVICE, "hipEventCreate failed");
      g_prof_pool.emplace_back(a, b);
    }
  }
  g_prof_kernel = kernel_id;
  return MOE_OK;
}

moe_status moe_profile_read(double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  moe_status st = MOE_OK;
  for (size_t i = 0; i < g_prof_used; ++i) {
    float ms = 0.0f;
    if (hipEventSynchronize(g_prof_pool[i].second) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof_pool[i].first, g_prof_pool[i].second) != hipSuccess)
      st = fail(MOE_ERR_DEVICE, "event timing failed");
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = static_cast<int64_t>(g_prof_used);
  g_prof_used = 0;
  return st;
}

}  // extern "C"
