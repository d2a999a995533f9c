"""Oracle against the brute-force checker on tiny inputs.

The brute force shares no code with the oracle: it applies every expert to
every token, finds KeepTopK by enumerating all k-subsets, gates with a literal
-infinity mask, and simulates capacity with per-expert counters. Agreement is
exact on integers and within 1e-12 on doubles.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _tiny(seed, T, H, F, N, k, order, noisy, cap, dtype, scale, tie_logits=False):
    w = synth.make_independent("tiny", seed, T, H, F, N, k, act=dtype, wt=dtype, order=order, noisy=noisy,
                               capacity=cap, out_scale=scale, wsig=0.5)
    if tie_logits:
        # quantise the router so that exact score ties are common
        w.Wg = np.round(w.Wg * 2.0).astype(np.float32)
        w.x = synth.f32_to_bf16(np.sign(w.f32("x"))) if dtype == "bf16" else np.sign(w.x).astype(np.float32)
    return w


def _compare(w, h_round):
    r = oracle.route(w)
    cap = oracle.capacity(w, r["topk_idx"])
    tokens = np.arange(w.T)
    y64, _ = oracle.combine_tokens(w, r["topk_idx"], r["topk_w"], cap["slot"], tokens, h_round=h_round)
    b = oracle.brute(w, h_round=h_round)
    assert np.array_equal(r["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(r["topk_w"], b["topk_w"], rtol=0, atol=1e-12)
    # dense gate from the oracle's compact form
    g = np.zeros((w.T, w.N))
    for t in range(w.T):
        g[t, r["topk_idx"][t]] = r["topk_w"][t]
    np.testing.assert_allclose(g, b["gate"], rtol=0, atol=1e-12)
    kept = (cap["slot"] >= 0).astype(np.int32)
    assert np.array_equal(kept, b["keep"])
    for t in range(w.T):
        for j in range(w.k):
            if cap["slot"][t, j] >= 0:
                e = r["topk_idx"][t, j]
                assert cap["slot"][t, j] - cap["offsets"][e] == b["rank"][t, j]
    assert np.array_equal(cap["counts"], b["load"])
    np.testing.assert_allclose(y64, b["y64"], rtol=0, atol=1e-12 * max(1.0, float(np.abs(b["y64"]).max(initial=0.0))))
    st = oracle.stats(w, r)
    assert np.array_equal(st["load"], b["load"])
    np.testing.assert_allclose(st["importance"], b["importance"], atol=1e-12)
    np.testing.assert_allclose(st["P"], b["P"], atol=1e-12)
    assert abs(st["balance"] - b["balance"]) < 1e-12


GRID = list(itertools.product([0, 1], [False, True], [-1, 0, 1, 3], ["f32", "bf16"]))


@pytest.mark.parametrize("gi", range(len(GRID)), ids=[f"{o}-{n}-{c}-{d}" for o, n, c, d in GRID])
def test_oracle_matches_brute(gi):
    order, noisy, cap, dtype = GRID[gi]
    rng = np.random.default_rng(1234 + gi)
    for s in range(32):
        T = int(rng.integers(0, 17))
        N = int(rng.integers(1, 7))
        k = int(rng.integers(1, N + 1))
        H = int(rng.integers(1, 9))
        F = int(rng.integers(1, 9))
        scale = float(rng.choice([1.0, N / k]))
        w = _tiny(10_000 + s, T, H, F, N, k, order, noisy, cap, dtype, scale)
        h_round = oracle.H_BF16 if dtype == "bf16" else oracle.H_F32
        _compare(w, h_round)


@pytest.mark.parametrize("order", [0, 1])
def test_oracle_matches_brute_exact_h(order):
    for s in range(200):
        w = _tiny(20_000 + s, 12, 6, 5, 5, 1 + s % 5, order, s % 2 == 1, -1 if s % 3 else 2, "f32", 1.0)
        _compare(w, oracle.H_EXACT)


@pytest.mark.parametrize("order", [0, 1])
def test_oracle_matches_brute_with_score_ties(order):
    """Quantised router and sign activations make many exact ties; both sides
    must break them to the lower expert index."""
    n_ties = 0
    for s in range(200):
        w = _tiny(30_000 + s, 16, 4, 3, 6, 1 + s % 6, order, False, -1 if s % 2 else 3, "f32", 1.0,
                  tie_logits=True)
        r = oracle.route(w)
        n_ties += int((r["min_gap"] == 0).sum())
        _compare(w, oracle.H_F32)
    assert n_ties > 100  # the test really exercises ties


def test_many_seeds_default_shape():
    """1000 seeds at one tiny shape, both orders, with and without capacity."""
    for s in range(1000):
        order = s % 2
        cap = [-1, 2, 5][s % 3]
        w = _tiny(40_000 + s, 16, 8, 8, 6, 2, order, s % 4 == 0, cap, "bf16", 3.0)
        _compare(w, oracle.H_BF16)
