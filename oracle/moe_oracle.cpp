/*
 * CPU ORACLE for the top-k MoE SwiGLU layer forward pass (test infrastructure
 * only; see moe_oracle.h for the sources and the rules of use).
 *
 * Each function restates one step of the method as its plain definition, in
 * double precision, one token at a time. Comments name the page and the
 * section or equation each step follows.
 */
#include "moe_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

/* exact decode of one stored element */
inline double load_val(const void* base, int32_t dtype, int64_t i) {
  if (dtype == ORC_BF16) {
    uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return static_cast<double>(f);
  }
  return static_cast<double>(static_cast<const float*>(base)[i]);
}

bool cfg_ok(const oracle_cfg* c) {
  if (!c) return false;
  if (c->T < 0 || c->H < 1 || c->F < 1 || c->N < 1 || c->k < 1 || c->k > c->N) return false;
  if (c->order != ORC_KEEPTOPK_SOFTMAX && c->order != ORC_SOFTMAX_TOPK) return false;
  if (c->h_round < ORC_H_EXACT || c->h_round > ORC_H_BF16) return false;
  return true;
}

/* Run body(i) for i in [0, n) on up to nthreads threads; each i is independent,
 * so the result does not depend on the thread count. */
template <class Fn>
void for_tokens(int64_t n, int32_t nthreads, Fn body) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  int64_t nt = std::min<int64_t>(nthreads, n);
  std::vector<std::thread> pool;
  for (int64_t w = 0; w < nt; ++w)
    pool.emplace_back([=, &body]() {
      for (int64_t i = w; i < n; i += nt) body(i);
    });
  for (auto& th : pool) th.join();
}

/* Order of expert indices by score descending, ties to the lower index. */
void sort_scores(const float* Hrow, int32_t N, std::vector<int32_t>& ord) {
  ord.resize(N);
  for (int32_t i = 0; i < N; ++i) ord[i] = i;
  std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) {
    return Hrow[a] > Hrow[b];  // stable: equal scores keep ascending index
  });
}

/* E = down(round(SiLU(gate x) * up x)) for one token row xd[H]. */
void expert_apply(const oracle_cfg* c, const double* xd, const void* Wgate, const void* Wup,
                  const void* Wdown, int32_t e, double* hbuf, double* E) {
  const int64_t H = c->H, F = c->F;
  const int64_t wbase = static_cast<int64_t>(e) * F * H;
  /* [V2] code example, Expert.forward: gate_proj, SiLU, times up_proj */
  for (int64_t f = 0; f < F; ++f) {
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      g += xd[h] * load_val(Wgate, c->w_dtype, wbase + f * H + h);
      u += xd[h] * load_val(Wup, c->w_dtype, wbase + f * H + h);
    }
    double a = oracle_silu(g) * u;
    if (c->h_round == ORC_H_BF16) a = oracle_round_bf16(a);
    else if (c->h_round == ORC_H_F32) a = oracle_round_f32(a);
    hbuf[f] = a;
  }
  /* down_proj */
  for (int64_t o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int64_t f = 0; f < F; ++f) acc += hbuf[f] * load_val(Wdown, c->w_dtype, wbase + o * F + f);
    E[o] = acc;
  }
}

}  // namespace

extern "C" {

double oracle_round_f32(double v) { return static_cast<double>(static_cast<float>(v)); }

/* Round to the nearest bf16 value (8 significant bits, fp32 exponent range),
 * ties to even, overflow to infinity. */
double oracle_round_bf16(double v) {
  if (std::isnan(v) || std::isinf(v) || v == 0.0) return v;
  const double a = std::fabs(v);
  int ex;
  std::frexp(a, &ex);                     /* a = m * 2^ex, m in [0.5, 1) */
  int q = ex - 8;                         /* spacing of 8-bit significands at this exponent */
  if (q < -133) q = -133;                 /* bf16 subnormal spacing 2^-133 */
  double r = std::nearbyint(std::ldexp(a, -q));  /* default mode: nearest, ties to even */
  double out = std::ldexp(r, q);
  if (out >= std::ldexp(1.0, 128)) out = std::numeric_limits<double>::infinity();
  return std::copysign(out, v);
}

/* SiLU(z) = z * sigmoid(z) ([V2] code example, nn.SiLU) */
double oracle_silu(double z) { return z / (1.0 + std::exp(-z)); }

/* Softplus(z) = ln(1 + e^z), written in the overflow-free form
 * max(z, 0) + ln(1 + e^-|z|) ([UP] section 3, noisy top-k router) */
double oracle_softplus(double z) { return std::max(z, 0.0) + std::log1p(std::exp(-std::fabs(z))); }

int oracle_route(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                 float* logits, float* Hv, int32_t* topk_idx, double* topk_w, double* min_gap) {
  if (!cfg_ok(c)) return -1;
  if (c->T > 0 && (!x || !Wg || !logits || !Hv || !topk_idx || !topk_w || !min_gap)) return -2;
  if (c->noisy && c->T > 0 && (!Wn || !eps)) return -2;
  const int64_t T = c->T, H = c->H, N = c->N, k = c->k;
  std::vector<double> xd(H), lg(N), nz(N);
  std::vector<int32_t> ord;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
    /* [UP] section 3: (x . W_g)_i, and (x . W_noise)_i when noisy */
    for (int64_t i = 0; i < N; ++i) {
      double a = 0.0, b = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        a += xd[h] * static_cast<double>(Wg[h * N + i]);
        if (c->noisy) b += xd[h] * static_cast<double>(Wn[h * N + i]);
      }
      lg[i] = a;
      nz[i] = b;
    }
    float* Hrow = Hv + t * N;
    for (int64_t i = 0; i < N; ++i) {
      logits[t * N + i] = static_cast<float>(lg[i]);
      /* H_i = (x W_g)_i + StandardNormal() * Softplus((x W_noise)_i); the normal
       * draw is the input eps[t,i] */
      double hv = lg[i];
      if (c->noisy) hv += static_cast<double>(eps[t * N + i]) * oracle_softplus(nz[i]);
      /* the pages leave non-numbers open; a NaN score is read as -inf: it
       * never outranks a number and adds 0 to every softmax denominator */
      if (std::isnan(hv)) hv = -std::numeric_limits<double>::infinity();
      Hrow[i] = static_cast<float>(hv);
    }
    /* KeepTopK ([UP] section 3): the k largest scores, ties to the lower index */
    sort_scores(Hrow, static_cast<int32_t>(N), ord);
    for (int64_t j = 0; j < k; ++j) topk_idx[t * k + j] = ord[j];
    double gap = std::numeric_limits<double>::infinity();
    const int64_t last = std::min<int64_t>(k + 1, N);
    for (int64_t j = 0; j + 1 < last; ++j)
      gap = std::min(gap, static_cast<double>(Hrow[ord[j]]) - static_cast<double>(Hrow[ord[j + 1]]));
    min_gap[t] = gap;
    const double hmax = Hrow[ord[0]];
    if (c->order == ORC_KEEPTOPK_SOFTMAX) {
      /* Mixtral order: Softmax over KeepTopK(H); the -inf entries contribute 0,
       * so the softmax runs over the k kept scores */
      double den = 0.0;
      for (int64_t j = 0; j < k; ++j) den += std::exp(static_cast<double>(Hrow[ord[j]]) - hmax);
      for (int64_t j = 0; j < k; ++j)
        topk_w[t * k + j] = std::exp(static_cast<double>(Hrow[ord[j]]) - hmax) / den;
    } else {
      /* ST order ([UP] section 5): softmax over all N scores, then keep the
       * top-k probabilities as they are (no renormalisation) */
      double den = 0.0;
      for (int64_t i = 0; i < N; ++i) den += std::exp(static_cast<double>(Hrow[i]) - hmax);
      for (int64_t j = 0; j < k; ++j)
        topk_w[t * k + j] = std::exp(static_cast<double>(Hrow[ord[j]]) - hmax) / den;
    }
  }
  return 0;
}

int oracle_stats(const oracle_cfg* c, const float* logits, const int32_t* topk_idx, const double* topk_w,
                 int64_t* load, double* importance, double* P, double* f, double* balance,
                 double* balance_code) {
  if (!cfg_ok(c)) return -1;
  if (!load || !importance || !P || !f || !balance || !balance_code) return -2;
  const int64_t T = c->T, N = c->N, k = c->k;
  for (int64_t i = 0; i < N; ++i) {
    load[i] = 0;
    importance[i] = 0.0;
    P[i] = 0.0;
  }
  /* Gate Load: assignments per expert before capacity; Gate Importance: sum
   * of the gate weights given to it */
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      load[e] += 1;
      importance[e] += topk_w[t * k + j];
    }
  /* P_i: mean over tokens of the softmax of the clean logits ([V2] code
   * example uses F.softmax(logits) without the noise) */
  std::vector<double> p(N);
  for (int64_t t = 0; t < T; ++t) {
    double m = logits[t * N];
    for (int64_t i = 1; i < N; ++i) m = std::max(m, static_cast<double>(logits[t * N + i]));
    double den = 0.0;
    for (int64_t i = 0; i < N; ++i) den += (p[i] = std::exp(static_cast<double>(logits[t * N + i]) - m));
    for (int64_t i = 0; i < N; ++i) P[i] += p[i] / den;
  }
  double bal = 0.0, tot_imp = 0.0, pm_dot_freq = 0.0;
  for (int64_t i = 0; i < N; ++i) tot_imp += importance[i];
  for (int64_t i = 0; i < N; ++i) {
    P[i] = T > 0 ? P[i] / static_cast<double>(T) : 0.0;
    /* f_i: fraction of the T*k assignments routed to expert i */
    f[i] = T > 0 ? static_cast<double>(load[i]) / static_cast<double>(T * k) : 0.0;
    /* [V2] gating section: L = lambda * sum_i f_i P_i (lambda left to the caller) */
    bal += f[i] * P[i];
    pm_dot_freq += (importance[i] / (tot_imp + 1e-6)) * P[i];
  }
  *balance = bal;
  *balance_code = pm_dot_freq * static_cast<double>(N);
  return 0;
}

int oracle_smooth_load(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                       double* smooth_load) {
  if (!cfg_ok(c) || !c->noisy) return -1;
  if (!smooth_load) return -2;
  if (c->T > 0 && (!x || !Wg || !Wn || !eps)) return -2;
  const int64_t T = c->T, H = c->H, N = c->N, k = c->k;
  std::vector<double> xd(H), lg(N), sp(N);
  std::vector<float> hv(N), others;
  for (int64_t i = 0; i < N; ++i) smooth_load[i] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
    for (int64_t i = 0; i < N; ++i) {
      double a = 0.0, b = 0.0;
      for (int64_t h = 0; h < H; ++h) {
        a += xd[h] * static_cast<double>(Wg[h * N + i]);
        b += xd[h] * static_cast<double>(Wn[h * N + i]);
      }
      lg[i] = static_cast<double>(static_cast<float>(a)); /* the fp32 clean logit */
      sp[i] = oracle_softplus(b);
      /* the selection score H_i of [UP] section 3, as oracle_route stores it
       * (fp32; a NaN read as -inf) */
      double s = a + static_cast<double>(eps[t * N + i]) * sp[i];
      if (std::isnan(s)) s = -std::numeric_limits<double>::infinity();
      hv[i] = static_cast<float>(s);
    }
    for (int64_t i = 0; i < N; ++i) {
      /* kth_excluding: the k-th highest score among the other experts */
      others.clear();
      for (int64_t j = 0; j < N; ++j)
        if (j != i) others.push_back(hv[j]);
      std::sort(others.begin(), others.end(), [](float a, float b) { return a > b; });
      const double thr = static_cast<int64_t>(others.size()) >= k ? static_cast<double>(others[k - 1])
                                                                  : -std::numeric_limits<double>::infinity();
      /* Phi(z) = erfc(-z / sqrt(2)) / 2 */
      const double z = (lg[i] - thr) / sp[i];
      smooth_load[i] += 0.5 * std::erfc(-z / std::sqrt(2.0));
    }
  }
  return 0;
}

int oracle_capacity(const oracle_cfg* c, const int32_t* topk_idx, int64_t* counts, int64_t* kept,
                    int64_t* offsets, int64_t* slot, int64_t* row_token) {
  if (!cfg_ok(c)) return -1;
  if (!counts || !kept || !offsets) return -2;
  const int64_t T = c->T, N = c->N, k = c->k;
  std::vector<int64_t> rank(static_cast<size_t>(T * k));
  for (int64_t i = 0; i < N; ++i) counts[i] = 0;
  /* [UP] section 3, capacity factor: each expert takes its assignments in
   * token order; the ones past its capacity overflow and are dropped */
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      rank[t * k + j] = counts[e]++;
    }
  for (int64_t i = 0; i < N; ++i) kept[i] = c->capacity < 0 ? counts[i] : std::min(counts[i], c->capacity);
  offsets[0] = 0;
  for (int64_t i = 0; i < N; ++i) offsets[i + 1] = offsets[i] + kept[i];
  for (int64_t r = 0; r < T * k; ++r) row_token[r] = -1;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      int64_t rk = rank[t * k + j];
      if (rk < kept[e]) {
        slot[t * k + j] = offsets[e] + rk;
        row_token[offsets[e] + rk] = t;
      } else {
        slot[t * k + j] = -1;
      }
    }
  return 0;
}

int oracle_expert_rows(const oracle_cfg* c, const void* x, const void* Wgate, const void* Wup,
                       const void* Wdown, int32_t e, const int64_t* tokens, int64_t n, int32_t nthreads,
                       double* h_out, double* E_out) {
  if (!cfg_ok(c)) return -1;
  if (e < 0 || e >= c->N) return -1;
  if (n > 0 && (!x || !Wgate || !Wup || !Wdown || !tokens || !E_out)) return -2;
  const int64_t H = c->H, F = c->F;
  for_tokens(n, nthreads, [&](int64_t i) {
    std::vector<double> xd(H), hb(F);
    const int64_t t = tokens[i];
    for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
    expert_apply(c, xd.data(), Wgate, Wup, Wdown, e, hb.data(), E_out + i * H);
    if (h_out)
      for (int64_t f = 0; f < F; ++f) h_out[i * F + f] = hb[f];
  });
  return 0;
}

int oracle_combine_tokens(const oracle_cfg* c, const void* x, const void* Wgate, const void* Wup,
                          const void* Wdown, const int32_t* topk_idx, const double* topk_w,
                          const int64_t* slot, const int64_t* tokens, int64_t n, int32_t nthreads,
                          double* y64, float* y32) {
  if (!cfg_ok(c)) return -1;
  if (n > 0 && (!x || !Wgate || !Wup || !Wdown || !topk_idx || !topk_w || !slot || !tokens)) return -2;
  const int64_t H = c->H, F = c->F, k = c->k;
  for_tokens(n, nthreads, [&](int64_t i) {
    std::vector<double> xd(H), hb(F), E(H), acc(H, 0.0);
    const int64_t t = tokens[i];
    for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
    /* [UP] section 3: y = sum_i G(x)_i E_i(x) over the kept experts, in the
     * token's top-k order; an overflowed slot skips its expert and adds 0 */
    for (int64_t j = 0; j < k; ++j) {
      if (slot[t * k + j] < 0) continue;
      expert_apply(c, xd.data(), Wgate, Wup, Wdown, topk_idx[t * k + j], hb.data(), E.data());
      const double w = topk_w[t * k + j];
      for (int64_t h = 0; h < H; ++h) acc[h] += w * E[h];
    }
    /* [V2] rescaling section: y = (N/k) * sum G_i E_i, with s given */
    for (int64_t h = 0; h < H; ++h) {
      const double y = c->out_scale * acc[h];
      if (y64) y64[i * H + h] = y;
      if (y32) y32[i * H + h] = static_cast<float>(y);
    }
  });
  return 0;
}

int oracle_combine_rows(const oracle_cfg* c, const double* topk_w, const int64_t* slot, const int64_t* tokens,
                        int64_t n, const double* E, double* y64, float* y32) {
  if (!cfg_ok(c)) return -1;
  if (n > 0 && (!topk_w || !slot || !tokens || !E)) return -2;
  const int64_t H = c->H, k = c->k;
  std::vector<double> acc(H);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = tokens[i];
    std::fill(acc.begin(), acc.end(), 0.0);
    /* [UP] section 3: y = sum_i G(x)_i E_i(x) over the kept experts, in the
     * token's top-k order; an overflowed slot adds 0 */
    for (int64_t j = 0; j < k; ++j) {
      if (slot[t * k + j] < 0) continue;
      const double w = topk_w[t * k + j];
      const double* Ej = E + (i * k + j) * H;
      for (int64_t h = 0; h < H; ++h) acc[h] += w * Ej[h];
    }
    /* [V2] rescaling section: y = s * sum G_i E_i */
    for (int64_t h = 0; h < H; ++h) {
      const double y = c->out_scale * acc[h];
      if (y64) y64[i * H + h] = y;
      if (y32) y32[i * H + h] = static_cast<float>(y);
    }
  }
  return 0;
}

int oracle_residual_combine_rows(const oracle_cfg* c, const double* topk_w, const int64_t* slot,
                                 const int64_t* tokens, int64_t n, const double* E, const double* R, double* y64,
                                 float* y32) {
  if (!cfg_ok(c)) return -1;
  if (n > 0 && (!topk_w || !slot || !tokens || !E || !R)) return -2;
  const int64_t H = c->H, k = c->k;
  std::vector<double> acc(H);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = tokens[i];
    std::fill(acc.begin(), acc.end(), 0.0);
    /* the routed part: sum of the kept experts' gate-weighted outputs, in the
     * token's top-k order */
    for (int64_t j = 0; j < k; ++j) {
      if (slot[t * k + j] < 0) continue;
      const double w = topk_w[t * k + j];
      const double* Ej = E + (i * k + j) * H;
      for (int64_t h = 0; h < H; ++h) acc[h] += w * Ej[h];
    }
    /* the shared slice is always active and is not rescaled; s applies to
     * the routed sum */
    for (int64_t h = 0; h < H; ++h) {
      const double y = R[i * H + h] + c->out_scale * acc[h];
      if (y64) y64[i * H + h] = y;
      if (y32) y32[i * H + h] = static_cast<float>(y);
    }
  }
  return 0;
}

int oracle_backward(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                    const void* Wgate, const void* Wup, const void* Wdown, const float* dy, double d_balance,
                    int32_t nthreads, double* dx, double* dWg, double* dWn, double* dWgate, double* dWup,
                    double* dWdown) {
  if (!cfg_ok(c)) return -1;
  if (!dx || !dWg || !dWn || !dWgate || !dWup || !dWdown) return -2;
  if (c->T > 0 && (!x || !Wg || !Wgate || !Wup || !Wdown || !dy)) return -2;
  if (c->noisy && c->T > 0 && (!Wn || !eps)) return -2;
  const int64_t T = c->T, H = c->H, F = c->F, N = c->N, k = c->k;
  const bool bf = c->h_round == ORC_H_BF16;
  auto rnd = [&](double v) { return bf ? oracle_round_bf16(v) : v; };
  std::fill(dx, dx + T * H, 0.0);
  std::fill(dWg, dWg + H * N, 0.0);
  std::fill(dWn, dWn + H * N, 0.0);
  std::fill(dWgate, dWgate + N * F * H, 0.0);
  std::fill(dWup, dWup + N * F * H, 0.0);
  std::fill(dWdown, dWdown + N * H * F, 0.0);
  if (T == 0) return 0;

  /* the forward's routing, capacity and gate weights */
  std::vector<float> logits(T * N), Hv(T * N);
  std::vector<int32_t> idx(T * k);
  std::vector<double> w(T * k), gap(T);
  oracle_route(c, x, Wg, Wn, eps, logits.data(), Hv.data(), idx.data(), w.data(), gap.data());
  std::vector<int64_t> counts(N), kept(N), offsets(N + 1), slot(T * k), row_token(T * k);
  oracle_capacity(c, idx.data(), counts.data(), kept.data(), offsets.data(), slot.data(), row_token.data());

  /* The experts, one expert per task: its kept rows in token order, so each
   * weight-gradient element sums its rows in token order whatever the thread
   * count. Each row leaves dw (its gate weight's gradient) and its share of
   * dx; the token's shares are added in slot order below. */
  std::vector<double> dwv(T * k, 0.0), dxp(T * k * H, 0.0);
  for_tokens(N, nthreads, [&](int64_t e) {
    std::vector<double> xd(H), g(F), u(F), hh(F), E(H), dE(H), dh(F), dg(F), du(F);
    const int64_t wb = e * F * H;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < k; ++j) {
        /* a dropped slot adds nothing to y: no gradient */
        if (idx[t * k + j] != e || slot[t * k + j] < 0) continue;
        for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
        /* forward of expert e on this token ([V2] code example, Expert) */
        for (int64_t f = 0; f < F; ++f) {
          double a = 0.0, b = 0.0;
          for (int64_t h = 0; h < H; ++h) {
            a += xd[h] * load_val(Wgate, c->w_dtype, wb + f * H + h);
            b += xd[h] * load_val(Wup, c->w_dtype, wb + f * H + h);
          }
          g[f] = a;
          u[f] = b;
          double v = oracle_silu(a) * b;
          if (c->h_round == ORC_H_BF16) v = oracle_round_bf16(v);
          else if (c->h_round == ORC_H_F32) v = oracle_round_f32(v);
          hh[f] = v;
        }
        for (int64_t o = 0; o < H; ++o) {
          double acc = 0.0;
          for (int64_t f = 0; f < F; ++f) acc += hh[f] * load_val(Wdown, c->w_dtype, wb + o * F + f);
          E[o] = acc;
        }
        /* y_t = s sum_j w_j E_j: dw_j = s <dy_t, E_j>, dE_j = s w_j dy_t */
        double d = 0.0;
        for (int64_t o = 0; o < H; ++o) d += static_cast<double>(dy[t * H + o]) * E[o];
        dwv[t * k + j] = c->out_scale * d;
        for (int64_t o = 0; o < H; ++o) dE[o] = rnd(c->out_scale * w[t * k + j] * static_cast<double>(dy[t * H + o]));
        /* down projection: dWdown_e += dE h^T, dh = Wdown_e^T dE */
        for (int64_t o = 0; o < H; ++o)
          for (int64_t f = 0; f < F; ++f) dWdown[wb + o * F + f] += dE[o] * hh[f];
        for (int64_t f = 0; f < F; ++f) {
          double acc = 0.0;
          for (int64_t o = 0; o < H; ++o) acc += dE[o] * load_val(Wdown, c->w_dtype, wb + o * F + f);
          dh[f] = acc;
        }
        /* h = SiLU(g) u: du = dh SiLU(g), dg = dh u SiLU'(g) with
         * SiLU'(g) = sigma(g) (1 + g (1 - sigma(g))) */
        for (int64_t f = 0; f < F; ++f) {
          const double sg = 1.0 / (1.0 + std::exp(-g[f]));
          du[f] = rnd(dh[f] * oracle_silu(g[f]));
          dg[f] = rnd(dh[f] * u[f] * sg * (1.0 + g[f] * (1.0 - sg)));
        }
        /* gate and up projections: dW += d outer x; this row's dx share W^T d */
        double* dxr = dxp.data() + (t * k + j) * H;
        for (int64_t f = 0; f < F; ++f)
          for (int64_t h = 0; h < H; ++h) {
            dWgate[wb + f * H + h] += dg[f] * xd[h];
            dWup[wb + f * H + h] += du[f] * xd[h];
            dxr[h] += dg[f] * load_val(Wgate, c->w_dtype, wb + f * H + h) +
                      du[f] * load_val(Wup, c->w_dtype, wb + f * H + h);
          }
      }
  });

  /* per token: the gate weights back to the scores and the router logits */
  std::vector<double> dlog(T * N, 0.0), dnv(T * N, 0.0);
  for_tokens(T, nthreads, [&](int64_t t) {
    std::vector<double> dH(N, 0.0), p(N), dp(N, 0.0), xd(H);
    const double* dw = dwv.data() + t * k;
    /* [UP] section 3, G = Softmax(KeepTopK(H)). Mixtral: w = softmax over
     * the kept k scores, dH_j = w_j (dw_j - sum w dw); ST ([UP] section 5):
     * w_j = p_{idx_j}, p = softmax over all N scores, dp is dw at the kept
     * indices and 0 elsewhere, dH = p (dp - <p, dp>) */
    const float* Hrow = Hv.data() + t * N;
    if (c->order == ORC_KEEPTOPK_SOFTMAX) {
      double sdot = 0.0;
      for (int64_t j = 0; j < k; ++j) sdot += w[t * k + j] * dw[j];
      for (int64_t j = 0; j < k; ++j) dH[idx[t * k + j]] += w[t * k + j] * (dw[j] - sdot);
    } else {
      double hmax = -std::numeric_limits<double>::infinity();
      for (int64_t i = 0; i < N; ++i) hmax = std::max(hmax, static_cast<double>(Hrow[i]));
      double den = 0.0;
      for (int64_t i = 0; i < N; ++i) den += (p[i] = std::exp(static_cast<double>(Hrow[i]) - hmax));
      for (int64_t i = 0; i < N; ++i) p[i] /= den;
      for (int64_t j = 0; j < k; ++j) dp[idx[t * k + j]] += dw[j];
      double sdot = 0.0;
      for (int64_t i = 0; i < N; ++i) sdot += p[i] * dp[i];
      for (int64_t i = 0; i < N; ++i) dH[i] = p[i] * (dp[i] - sdot);
    }
    /* balance = sum_i f_i P_i with P_i = mean over tokens of softmax(clean
     * logits) ([V2] gating section): d balance / d logit_t,m =
     * (1/T) p_m (f_m - <f, p>), p = softmax(logits_t) */
    double m = -std::numeric_limits<double>::infinity();
    for (int64_t i = 0; i < N; ++i) m = std::max(m, static_cast<double>(logits[t * N + i]));
    double den = 0.0;
    for (int64_t i = 0; i < N; ++i) den += (p[i] = std::exp(static_cast<double>(logits[t * N + i]) - m));
    double fp = 0.0;
    for (int64_t i = 0; i < N; ++i) {
      p[i] /= den;
      fp += (static_cast<double>(counts[i]) / static_cast<double>(T * k)) * p[i];
    }
    for (int64_t i = 0; i < N; ++i)
      dlog[t * N + i] = dH[i] + d_balance / static_cast<double>(T) * p[i] *
                                    (static_cast<double>(counts[i]) / static_cast<double>(T * k) - fp);
    /* H = logits + eps * Softplus(x W_noise): d/dn = dH eps sigmoid(n) */
    for (int64_t h = 0; h < H; ++h) xd[h] = load_val(x, c->x_dtype, t * H + h);
    if (c->noisy) {
      for (int64_t i = 0; i < N; ++i) {
        double b = 0.0;
        for (int64_t h = 0; h < H; ++h) b += xd[h] * static_cast<double>(Wn[h * N + i]);
        dnv[t * N + i] = dH[i] * static_cast<double>(eps[t * N + i]) / (1.0 + std::exp(-b));
      }
    }
    /* dx: the slots' shares in slot order, then the router terms
     * (logits = x W_g, noise logits = x W_noise) */
    for (int64_t h = 0; h < H; ++h) {
      double v = 0.0;
      for (int64_t j = 0; j < k; ++j) v += dxp[(t * k + j) * H + h];
      for (int64_t i = 0; i < N; ++i) {
        v += dlog[t * N + i] * static_cast<double>(Wg[h * N + i]);
        if (c->noisy) v += dnv[t * N + i] * static_cast<double>(Wn[h * N + i]);
      }
      dx[t * H + h] = v;
    }
  });
  /* router weights: dWg = x^T dlog, dWn = x^T dn, each element over the
   * tokens in order */
  for_tokens(H, nthreads, [&](int64_t h) {
    for (int64_t t = 0; t < T; ++t) {
      const double xv = load_val(x, c->x_dtype, t * H + h);
      for (int64_t i = 0; i < N; ++i) {
        dWg[h * N + i] += xv * dlog[t * N + i];
        if (c->noisy) dWn[h * N + i] += xv * dnv[t * N + i];
      }
    }
  });
  return 0;
}

}  // extern "C"
