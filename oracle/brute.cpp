/*
 * BRUTE-FORCE CHECKER for the CPU oracle (test infrastructure only).
 *
 * For tiny inputs it evaluates the layer straight from the equations, with no
 * code shared with moe_oracle.cpp:
 *   - every expert is applied to every token (dense), then the gate decides;
 *   - KeepTopK is found by enumerating every k-subset of the N scores and
 *     taking the largest sum, ties to the lexicographically smallest index
 *     set ("Llama 3 Meets MoE" review, section 3, KeepTopK);
 *   - the Mixtral gate is a softmax over all N entries of the masked vector
 *     with literal -infinity outside the kept set (same section, G(x));
 *     the ST gate is a softmax over all N scores, zeroed outside the set
 *     (section 5, router ablation);
 *   - capacity is simulated with one running counter per expert, tokens in
 *     order (section 3, capacity factor);
 *   - bf16 rounding uses a quotient/remainder construction instead of the
 *     oracle's frexp/nearbyint one.
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "moe_oracle.h"

namespace {

double brute_decode(const void* p, int32_t dt, int64_t i) {
  if (dt == ORC_BF16) {
    uint16_t b = static_cast<const uint16_t*>(p)[i];
    uint32_t w = static_cast<uint32_t>(b) * 65536u;
    float f;
    std::memcpy(&f, &w, sizeof f);
    return f;
  }
  return static_cast<const float*>(p)[i];
}

double brute_bf16(double v) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  double a = std::fabs(v);
  int e = std::ilogb(a);            /* a in [2^e, 2^(e+1)) */
  if (e < -126) e = -126;           /* below the normal range the spacing stays 2^-133 */
  double ulp = std::ldexp(1.0, e - 7);
  double q = std::floor(a / ulp);
  double rem = a - q * ulp;
  double half = 0.5 * ulp;
  if (rem > half || (rem == half && std::fmod(q, 2.0) != 0.0)) q += 1.0;
  double r = q * ulp;
  if (r >= std::ldexp(1.0, 128)) r = std::numeric_limits<double>::infinity();
  return v < 0 ? -r : r;
}

double brute_round_h(const oracle_cfg* c, double a) {
  if (c->h_round == ORC_H_BF16) return brute_bf16(a);
  if (c->h_round == ORC_H_F32) return static_cast<double>(static_cast<float>(a));
  return a;
}

double brute_softplus(double z) { return z > 30.0 ? z + std::log1p(std::exp(-z)) : std::log(1.0 + std::exp(z)); }

double brute_sigmoid_times(double z) { return z * (1.0 / (1.0 + std::exp(-z))); }

int popcount32(uint32_t m) {
  int n = 0;
  for (; m; m &= m - 1) ++n;
  return n;
}

/* true if sorted index list a is lexicographically smaller than b */
bool lex_less(const std::vector<int>& a, const std::vector<int>& b) {
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i] != b[i]) return a[i] < b[i];
  return false;
}

}  // namespace

extern "C" {

/* Outputs (all sized for the whole batch):
 *   idx [T,k] (kept set ordered by score descending, ties to lower index),
 *   w [T,k] gate weight of idx, gate [T,N] dense gate vector,
 *   keep [T,k] 1 if the assignment survives capacity, rank [T,k] its position
 *   in its expert's token-ordered queue, y [T,H] double,
 *   load [N], importance [N], P [N], balance. */
int brute_layer(const oracle_cfg* c, const void* x, const float* Wg, const float* Wn, const float* eps,
                const void* Wgate, const void* Wup, const void* Wdown, int32_t* idx, double* w,
                double* gate, int32_t* keep, int64_t* rank, double* y, int64_t* load, double* importance,
                double* P, double* balance) {
  if (!c || c->N > 20 || c->k < 1 || c->k > c->N) return -1;
  const int T = static_cast<int>(c->T), H = c->H, F = c->F, N = c->N, k = c->k;
  std::vector<double> xs(H), lg(N), hv(N), Eall(static_cast<size_t>(N) * H), hh(F);
  std::vector<int64_t> counter(N, 0);
  for (int i = 0; i < N; ++i) {
    load[i] = 0;
    importance[i] = 0;
    P[i] = 0;
  }
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) xs[h] = brute_decode(x, c->x_dtype, static_cast<int64_t>(t) * H + h);
    for (int i = 0; i < N; ++i) {
      double a = 0, b = 0;
      for (int h = 0; h < H; ++h) {
        a += xs[h] * Wg[h * N + i];
        if (c->noisy) b += xs[h] * Wn[h * N + i];
      }
      lg[i] = static_cast<float>(a);
      double s = a;
      if (c->noisy) s = a + eps[t * N + i] * brute_softplus(b);
      hv[i] = static_cast<float>(s);
    }
    /* enumerate all k-subsets */
    std::vector<int> best, cur;
    double best_sum = -std::numeric_limits<double>::infinity();
    bool have = false;
    for (uint32_t m = 0; m < (1u << N); ++m) {
      if (popcount32(m) != k) continue;
      cur.clear();
      double s = 0;
      for (int i = 0; i < N; ++i)
        if (m & (1u << i)) {
          cur.push_back(i);
          s += hv[i];
        }
      if (!have || s > best_sum || (s == best_sum && lex_less(cur, best))) {
        best = cur;
        best_sum = s;
        have = true;
      }
    }
    /* order the kept set: insertion sort by score desc, index asc */
    std::vector<int> ordk = best;
    for (size_t a = 1; a < ordk.size(); ++a)
      for (size_t b = a; b > 0; --b) {
        int p = ordk[b - 1], q = ordk[b];
        bool swap = hv[q] > hv[p] || (hv[q] == hv[p] && q < p);
        if (!swap) break;
        ordk[b - 1] = q;
        ordk[b] = p;
      }
    /* dense gate */
    std::vector<double> g(N, 0.0);
    if (c->order == ORC_KEEPTOPK_SOFTMAX) {
      std::vector<double> masked(N, -std::numeric_limits<double>::infinity());
      for (int i : best) masked[i] = hv[i];
      double mx = -std::numeric_limits<double>::infinity();
      for (int i = 0; i < N; ++i) mx = masked[i] > mx ? masked[i] : mx;
      double den = 0;
      for (int i = 0; i < N; ++i) den += std::exp(masked[i] - mx);
      for (int i = 0; i < N; ++i) g[i] = std::exp(masked[i] - mx) / den;
    } else {
      double mx = hv[0];
      for (int i = 1; i < N; ++i) mx = hv[i] > mx ? hv[i] : mx;
      double den = 0;
      for (int i = 0; i < N; ++i) den += std::exp(hv[i] - mx);
      for (int i : best) g[i] = std::exp(hv[i] - mx) / den;
    }
    for (int i = 0; i < N; ++i) gate[t * N + i] = g[i];
    /* clean-logit softmax for P */
    {
      double mx = lg[0];
      for (int i = 1; i < N; ++i) mx = lg[i] > mx ? lg[i] : mx;
      double den = 0;
      for (int i = 0; i < N; ++i) den += std::exp(lg[i] - mx);
      for (int i = 0; i < N; ++i) P[i] += std::exp(lg[i] - mx) / den;
    }
    /* capacity: running counter per expert, this token's experts in index order */
    std::vector<int> kept_here(N, 0);
    for (int i = 0; i < N; ++i) {
      bool in = false;
      for (int q : best) in = in || (q == i);
      if (!in) continue;
      counter[i] += 1;
      load[i] += 1;
      importance[i] += g[i];
      kept_here[i] = (c->capacity < 0 || counter[i] <= c->capacity) ? 1 : 0;
      for (int j = 0; j < k; ++j)
        if (ordk[j] == i) rank[t * k + j] = counter[i] - 1;
    }
    for (int j = 0; j < k; ++j) {
      idx[t * k + j] = ordk[j];
      w[t * k + j] = g[ordk[j]];
      keep[t * k + j] = kept_here[ordk[j]];
    }
    /* every expert on this token */
    for (int e = 0; e < N; ++e) {
      const int64_t base = static_cast<int64_t>(e) * F * H;
      for (int f = 0; f < F; ++f) {
        double gg = 0, uu = 0;
        for (int h = 0; h < H; ++h) {
          gg += xs[h] * brute_decode(Wgate, c->w_dtype, base + static_cast<int64_t>(f) * H + h);
          uu += xs[h] * brute_decode(Wup, c->w_dtype, base + static_cast<int64_t>(f) * H + h);
        }
        hh[f] = brute_round_h(c, brute_sigmoid_times(gg) * uu);
      }
      for (int o = 0; o < H; ++o) {
        double s = 0;
        for (int f = 0; f < F; ++f) s += hh[f] * brute_decode(Wdown, c->w_dtype, base + static_cast<int64_t>(o) * F + f);
        Eall[static_cast<size_t>(e) * H + o] = s;
      }
    }
    for (int o = 0; o < H; ++o) {
      double s = 0;
      for (int e = 0; e < N; ++e) s += (kept_here[e] ? g[e] : 0.0) * Eall[static_cast<size_t>(e) * H + o];
      y[static_cast<int64_t>(t) * H + o] = c->out_scale * s;
    }
  }
  double bal = 0;
  for (int i = 0; i < N; ++i) {
    if (T > 0) P[i] /= T;
    double fi = T > 0 ? static_cast<double>(load[i]) / (static_cast<double>(T) * k) : 0.0;
    bal += fi * P[i];
  }
  *balance = bal;
  return 0;
}

double brute_round_bf16(double v) { return brute_bf16(v); }

}  // extern "C"
