"""moe_route (router GEMM, noisy gate, KeepTopK, gates, statistics) against
the oracle: indices exact (near ties reported), gate weights, clean logits and
statistics within fp32 rounding."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_smooth_load, log, routing_flips, run_route

pytestmark = pytest.mark.gpu


def _ties():
    w = synth.make_independent("ties", 41, 200, 64, 16, 6, 2, wsig=0.5)
    w.Wg = np.round(w.Wg * 2.0).astype(np.float32)
    w.x = synth.f32_to_bf16(np.sign(w.f32("x")))
    return w


CASES = {
    "f32_n8k2": lambda: synth.make_split("f32_n8k2", 11, 300, 256, 8 * 24, 8, 2, act="f32", wt="f32"),
    "f32_noisy_n16k4_stats": lambda: synth.make_independent("f32_noisy", 24, 301, 256, 8, 16, 4, act="f32",
                                                            wt="f32", noisy=True, want_stats=True),
    "f32_noisy_keqn": lambda: synth.make_independent("f32_noisy_keqn", 25, 130, 128, 8, 4, 4, act="f32",
                                                     wt="f32", noisy=True, want_stats=True),
    "bf16_n8k2": lambda: synth.make_split("bf16_n8k2", 12, 333, 512, 8 * 16, 8, 2),
    "noisy_n16k4_stats": lambda: synth.make_split("noisy", 13, 517, 1024, 16 * 8, 16, 4, noisy=True,
                                                   want_stats=True),
    "st_order": lambda: synth.make_split("st", 14, 200, 256, 64, 8, 2, order=synth.ST, want_stats=True),
    "n6k3_unaligned_rows": lambda: synth.make_independent("n6", 15, 150, 136, 8, 6, 3),
    "n40k5": lambda: synth.make_independent("n40", 16, 90, 256, 8, 40, 5, want_stats=True),
    "n24k1": lambda: synth.make_independent("n24", 17, 77, 128, 8, 24, 1),
    "k_eq_n": lambda: synth.make_independent("keqn", 18, 64, 64, 8, 4, 4, order=synth.ST),
    "n1k1": lambda: synth.make_independent("n1", 19, 33, 64, 8, 1, 1),
    "n64k8_noisy": lambda: synth.make_independent("n64", 20, 40, 256, 8, 64, 8, noisy=True, want_stats=True),
    "exact_ties": _ties,
    # the matrix-core router's code paths: folded B operand with the noise
    # columns (N <= 4), folded with H past two LDS chunks (the chunk loop,
    # with a partial last chunk), and unfolded at 9..16 columns
    "fold_noisy_n4k2": lambda: synth.make_independent("fn4", 21, 100, 256, 8, 4, 2, noisy=True, want_stats=True),
    "fold_long_h": lambda: synth.make_independent("flh", 22, 50, 4360, 8, 8, 2),
    "n12k3": lambda: synth.make_independent("n12", 23, 120, 512, 8, 12, 3),
    "C1_full": synth.c1,
    "C2_full_routing": lambda: synth.make_split("C2_routing", 1002, 4096, 4096, 8 * 8, 8, 2, out_scale=4.0),
    "C3_full_routing": lambda: synth.make_split("C3_routing", 1003, 4096, 4096, 16 * 8, 16, 4, noisy=True,
                                                want_stats=True, out_scale=4.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_route_matches_oracle(name):
    w = CASES[name]()
    log(f"[route] {name} T={w.T} H={w.H} N={w.N} k={w.k} noisy={w.noisy} order={w.order}")
    g = run_route(w)
    ora = oracle.route(w)
    flips = routing_flips(g["topk_idx"], ora, name)
    if name == "exact_ties":
        assert not flips.any() and (ora["min_gap"] == 0).sum() > 20
    np.testing.assert_allclose(g["logits"], ora["logits"], rtol=0, atol=5e-6 * max(1.0, np.abs(ora["logits"]).max()))
    ok = ~flips
    np.testing.assert_allclose(g["topk_w"][ok], ora["topk_w"][ok], rtol=2e-6, atol=1e-7)
    if w.order == synth.MIXTRAL:
        np.testing.assert_allclose(g["topk_w"].sum(axis=1), 1.0, atol=1e-6)
    if w.want_stats:
        st = oracle.stats(w, ora)
        if not flips.any():
            assert np.array_equal(g["load"], st["load"])
        np.testing.assert_allclose(g["importance"], st["importance"], rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(g["P"], st["P"], rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(g["balance"][0], st["balance"], rtol=1e-5)
        if w.noisy:
            check_smooth_load(g["smooth_load"], w, name)


def test_route_skewed_decode_prefers_expert_zero():
    w = synth.make_independent("skew", 1005, 64, 4096, 8, 8, 2)
    synth.apply_skew(w, n_pref=32)
    g = run_route(w, want_logits=False)
    ora = oracle.route(w)
    routing_flips(g["topk_idx"], ora, "skew")
    frac = float(np.mean(g["topk_idx"][:, 0] == 0))
    log(f"  fraction of tokens whose top-1 is expert 0: {frac:.3f}")
    assert frac >= 0.5
