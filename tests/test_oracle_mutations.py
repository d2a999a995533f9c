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
]

PIN_FILES = ["tests/test_golden.py", "tests/test_oracle_pins.py", "tests/test_oracle_invariants.py",
             "tests/test_oracle_brute.py"]


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for {name} not found"
    d = tmp_path / "oracle_src"
    d.mkdir()
    for f in ("moe_oracle.h", "brute.cpp"):
        shutil.copy(os.path.join(ROOT, "oracle", f), d / f)
    (d / "moe_oracle.cpp").write_text(src.replace(orig, bad, 1))
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    so = str(tmp_path / "liboracle_mut.so")
    ob.build(out=so, sources_dir=str(d))
    env = dict(os.environ, MOE_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' survived every pin:\n{r.stdout[-2000:]}"
