"""The oracle's pins catch plausible mistakes.

Each case copies the oracle source, plants one mistake (a dropped term, a
wrong sign, a transposed operand, an off-by-one, a wrong tie rule, ...),
builds the copy on the side and runs the oracle's pin tests against it in a
subprocess. The pins must fail for every planted mistake. The mistakes are
planted only in the temporary copy, on the CPU.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.cpp")

# (name, original text, planted mistake)
MUTANTS = [
    ("drop_noise_term",
     "if (c->noisy) hv += static_cast<double>(eps[t * N + i]) * oracle_softplus(nz[i]);",
     "(void)nz;"),
    ("softplus_sign",
     "std::log1p(std::exp(-std::fabs(z)))", "std::log1p(std::exp(std::fabs(z)))"),
    ("silu_sign", "return z / (1.0 + std::exp(-z));", "return z / (1.0 + std::exp(z));"),
    ("ties_to_higher_index", "return Hrow[a] > Hrow[b];  // stable",
     "return Hrow[a] > Hrow[b] || (Hrow[a] == Hrow[b] && a > b);  // stable"),
    ("mixtral_softmax_over_all_n",
     "for (int64_t j = 0; j < k; ++j) den += std::exp(static_cast<double>(Hrow[ord[j]]) - hmax);",
     "for (int64_t j = 0; j < N; ++j) den += std::exp(static_cast<double>(Hrow[j]) - hmax);"),
    ("st_renormalised",
     "for (int64_t i = 0; i < N; ++i) den += std::exp(static_cast<double>(Hrow[i]) - hmax);",
     "for (int64_t i = 0; i < k; ++i) den += std::exp(static_cast<double>(Hrow[ord[i]]) - hmax);"),
    ("capacity_off_by_one", "if (rk < kept[e]) {", "if (rk <= kept[e] && offsets[e] + rk < T * k) {"),
    ("offsets_ignore_capacity", "offsets[i + 1] = offsets[i] + kept[i];",
     "offsets[i + 1] = offsets[i] + counts[i];"),
    ("down_proj_transposed", "load_val(Wdown, c->w_dtype, wbase + o * F + f)",
     "load_val(Wdown, c->w_dtype, wbase + (f * H + o) % (F * H))"),
    ("silu_drops_z_factor", "return z / (1.0 + std::exp(-z));",
     "return 1.0 / (1.0 + std::exp(-z));"),
    ("drop_out_scale", "const double y = c->out_scale * acc[h];", "const double y = acc[h];"),
    ("skip_h_rounding", "if (c->h_round == ORC_H_BF16) a = oracle_round_bf16(a);",
     "if (c->h_round == ORC_H_BF16) a = a;"),
    ("bf16_ties_away", "double r = std::nearbyint(std::ldexp(a, -q));",
     "double r = std::round(std::ldexp(a, -q));"),
    ("balance_f_over_T",
     "f[i] = T > 0 ? static_cast<double>(load[i]) / static_cast<double>(T * k) : 0.0;",
     "f[i] = T > 0 ? static_cast<double>(load[i]) / static_cast<double>(T) : 0.0;"),
    ("P_from_wrong_row", "den += (p[i] = std::exp(static_cast<double>(logits[t * N + i]) - m));",
     "den += (p[i] = std::exp(static_cast<double>(logits[(t * N + i + 1) % (T * N)]) - m));"),
    ("min_gap_misses_boundary", "const int64_t last = std::min<int64_t>(k + 1, N);",
     "const int64_t last = std::min<int64_t>(k, N);"),
    ("combine_drops_second_slot", "for (int64_t j = 0; j < k; ++j) {\n      if (slot[t * k + j] < 0) continue;",
     "for (int64_t j = 0; j < 1; ++j) {\n      if (slot[t * k + j] < 0) continue;"),
    ("logit_reads_wrong_column", "a += xd[h] * static_cast<double>(Wg[h * N + i]);",
     "a += xd[h] * static_cast<double>(Wg[h * N + (N - 1 - i)]);"),
    ("code_balance_uses_load", "pm_dot_freq += (importance[i] / (tot_imp + 1e-6)) * P[i];",
     "pm_dot_freq += (static_cast<double>(load[i]) / (T * k + 1e-6)) * P[i];"),
    ("code_balance_drops_times_n", "*balance_code = pm_dot_freq * static_cast<double>(N);",
     "*balance_code = pm_dot_freq;"),
    ("code_balance_drops_guard", "pm_dot_freq += (importance[i] / (tot_imp + 1e-6)) * P[i];",
     "pm_dot_freq += (importance[i] / tot_imp) * P[i];"),
    ("combine_rows_drops_scale", "const double y = c->out_scale * acc[h];\n      if (y64) y64[i * H + h] = y;\n      if (y32) y32[i * H + h] = static_cast<float>(y);\n    }\n  }\n  return 0;",
     "const double y = acc[h];\n      if (y64) y64[i * H + h] = y;\n      if (y32) y32[i * H + h] = static_cast<float>(y);\n    }\n  }\n  return 0;"),
    ("combine_rows_reads_wrong_slot", "const double* Ej = E + (i * k + j) * H;", "const double* Ej = E + (i * k) * H;"),
    ("smooth_uses_noisy_numerator", "const double z = (lg[i] - thr) / sp[i];",
     "const double z = (static_cast<double>(hv[i]) - thr) / sp[i];"),
    ("smooth_kth_includes_self", "if (j != i) others.push_back(hv[j]);", "others.push_back(hv[j]);"),
    ("smooth_phi_sign", "0.5 * std::erfc(-z / std::sqrt(2.0))", "0.5 * std::erfc(z / std::sqrt(2.0))"),
    ("smooth_no_sqrt2", "0.5 * std::erfc(-z / std::sqrt(2.0))", "0.5 * std::erfc(-z)"),
    ("residual_scaled_with_routed", "const double y = R[i * H + h] + c->out_scale * acc[h];",
     "const double y = c->out_scale * (R[i * H + h] + acc[h]);"),
    ("residual_dropped", "const double y = R[i * H + h] + c->out_scale * acc[h];",
     "const double y = c->out_scale * acc[h];"),
    ("residual_keeps_dropped_slots",
     "      if (slot[t * k + j] < 0) continue;\n      const double w = topk_w[t * k + j];\n      const double* Ej = E + (i * k + j) * H;\n      for (int64_t h = 0; h < H; ++h) acc[h] += w * Ej[h];\n    }\n    /* the shared",
     "      const double w = topk_w[t * k + j];\n      const double* Ej = E + (i * k + j) * H;\n      for (int64_t h = 0; h < H; ++h) acc[h] += w * Ej[h];\n    }\n    /* the shared"),
    ("bwd_silu_derivative_drops_term", "dg[f] = rnd(dh[f] * u[f] * sg * (1.0 + g[f] * (1.0 - sg)));",
     "dg[f] = rnd(dh[f] * u[f] * sg);"),
    ("bwd_mixtral_jacobian_drops_mean", "dH[idx[t * k + j]] += w[t * k + j] * (dw[j] - sdot);",
     "dH[idx[t * k + j]] += w[t * k + j] * dw[j];"),
    ("bwd_st_jacobian_drops_p", "for (int64_t i = 0; i < N; ++i) dH[i] = p[i] * (dp[i] - sdot);",
     "for (int64_t i = 0; i < N; ++i) dH[i] = dp[i] - sdot;"),
    ("bwd_balance_sign", "(static_cast<double>(counts[i]) / static_cast<double>(T * k) - fp);",
     "(fp - static_cast<double>(counts[i]) / static_cast<double>(T * k));"),
    ("bwd_noise_softplus_not_sigmoid", "dnv[t * N + i] = dH[i] * static_cast<double>(eps[t * N + i]) / (1.0 + std::exp(-b));",
     "dnv[t * N + i] = dH[i] * static_cast<double>(eps[t * N + i]) * oracle_softplus(b);"),
    ("bwd_dE_drops_scale", "dE[o] = rnd(c->out_scale * w[t * k + j] * static_cast<double>(dy[t * H + o]));",
     "dE[o] = rnd(w[t * k + j] * static_cast<double>(dy[t * H + o]));"),
    ("bwd_dw_drops_scale", "dwv[t * k + j] = c->out_scale * d;", "dwv[t * k + j] = d;"),
    ("bwd_dWdown_transposed", "for (int64_t f = 0; f < F; ++f) dWdown[wb + o * F + f] += dE[o] * hh[f];",
     "for (int64_t f = 0; f < F; ++f) dWdown[wb + f * H + o] += dE[o] * hh[f];"),
    ("bwd_dropped_slot_gets_gradient", "if (idx[t * k + j] != e || slot[t * k + j] < 0) continue;",
     "if (idx[t * k + j] != e) continue;"),
    ("bwd_dx_misses_router_term", "        v += dlog[t * N + i] * static_cast<double>(Wg[h * N + i]);",
     "        (void)0;"),
    ("nan_score_not_ranked_last",
     "if (std::isnan(hv)) hv = -std::numeric_limits<double>::infinity();", "(void)0;"),
]

PIN_FILES = ["tests/test_golden.py", "tests/test_oracle_pins.py", "tests/test_oracle_invariants.py",
             "tests/test_oracle_brute.py", "tests/test_oracle_backward.py"]


def _run_mutant(name, orig, bad, work):
    """Build the oracle with one planted mistake and run every pin against it
    in a subprocess; returns (returncode, output tail)."""
    src = open(SRC).read()
    if src.count(orig) < 1:
        return None, f"mutation anchor for {name} not found"
    d = os.path.join(work, name)
    os.makedirs(d, exist_ok=True)
    for f in ("moe_oracle.h", "brute.cpp"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(d, f))
    with open(os.path.join(d, "moe_oracle.cpp"), "w") as fh:
        fh.write(src.replace(orig, bad, 1))
    from oracle import build as ob
    so = os.path.join(d, "liboracle_mut.so")
    ob.build(out=so, sources_dir=d)
    env = dict(os.environ, MOE_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(request, tmp_path_factory):
    """Run the selected mutants' pin suites in parallel subprocesses (each is
    single-threaded), once per session."""
    wanted = {item.callspec.params["name"] for item in request.session.items
              if item.originalname == "test_pins_catch_planted_mistake"}
    sys.path.insert(0, ROOT)
    work = str(tmp_path_factory.mktemp("mutants"))
    jobs = [m for m in MUTANTS if m[0] in wanted]
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {m[0]: ex.submit(_run_mutant, m[0], m[1], m[2], work) for m in jobs}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, bad, mutant_results):
    rc, tail = mutant_results[name]
    assert rc is not None, tail
    assert rc != 0, f"planted mistake '{name}' survived every pin:\n{tail}"
