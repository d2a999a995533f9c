"""Pins of the oracle's scalar pieces and its router product against library
routines (torch, numpy) that are independent of the oracle's code."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch_on_fp32_values():
    lib = oracle.load()
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),          # fp32 subnormals
        np.array([3.3895313892515355e38, 3.39e38, -3.39e38, 1e-45, 0.0, -0.0], np.float32),
    ])
    # exact halfway cases: bf16 value + half a bf16 ulp, for even and odd lower bits
    base = torch.tensor([1.0, 1.0078125, 1.015625, 3.0, -5.5, 0.15625], dtype=torch.float32)
    half = torch.tensor([2.0 ** -8, 2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6, 2.0 ** -11], dtype=torch.float32)
    vals = np.concatenate([vals, (base + half).numpy(), (base - half).numpy()])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([lib.oracle_round_bf16(float(v)) for v in vals])
    same = (got == ref) | (np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref)))
    assert same.all(), vals[~same][:10]


def test_bf16_rounding_oracle_vs_brute_on_doubles():
    """The oracle (frexp / nearbyint) and the brute force (quotient and
    remainder) round arbitrary doubles the same way."""
    lib = oracle.load()
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 39, 20000),
                           rng.standard_normal(1000) * 1e-40])
    a = np.array([lib.oracle_round_bf16(float(v)) for v in vals])
    b = np.array([lib.brute_round_bf16(float(v)) for v in vals])
    assert np.array_equal(a, b)
    # a double just above a bf16 halfway point rounds up, unlike a double
    # rounding through fp32 would
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert lib.oracle_round_bf16(v) == 1.0078125


def test_silu_and_softplus_against_torch():
    lib = oracle.load()
    z = torch.linspace(-60.0, 60.0, 4001, dtype=torch.float64)
    silu = torch.nn.functional.silu(z).numpy()
    sp = torch.nn.functional.softplus(z, beta=1.0, threshold=1e9).numpy()
    for i, zz in enumerate(z.numpy()):
        assert math.isclose(lib.oracle_silu(float(zz)), silu[i], rel_tol=1e-14, abs_tol=1e-300)
        assert math.isclose(lib.oracle_softplus(float(zz)), sp[i], rel_tol=1e-14, abs_tol=1e-300)
    assert abs(lib.oracle_softplus(0.0) - math.log(2.0)) < 1e-16


def test_router_logits_are_the_fp32_rounded_matmul():
    """Clean logits equal fl32 of the exact product x.Wg (numpy float64 matmul,
    a different summation order: agreement to half an fp32 ulp)."""
    w = synth.make_split("t", 77, 64, 256, 64, 8, 2)
    r = oracle.route(w)
    exact = w.f32("x").astype(np.float64) @ w.Wg.astype(np.float64)
    err = np.abs(r["logits"].astype(np.float64) - exact)
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    assert np.all(err <= 0.5 * ulp * (1 + 1e-6) + 1e-30)


def test_noisy_scores_against_torch():
    """H = fl32(x.Wg + eps * softplus(x.Wn)) with torch float64 ops."""
    w = synth.make_split("t", 78, 32, 128, 32, 16, 4, noisy=True)
    r = oracle.route(w)
    x = torch.from_numpy(w.f32("x")).double()
    ref = (x @ torch.from_numpy(w.Wg).double()
           + torch.from_numpy(w.eps).double()
           * torch.nn.functional.softplus(x @ torch.from_numpy(w.Wn).double(), threshold=1e9))
    ref32 = ref.float().numpy()
    diff = np.abs(r["H"] - ref32)
    ulp = np.spacing(np.abs(ref32))
    assert np.all(diff <= ulp)  # at most one fp32 step from a different summation order
    assert (diff == 0).mean() > 0.95


def test_topk_and_gates_against_torch():
    """KeepTopK and the two gate orders against torch.topk / torch.softmax on
    the oracle's own fp32 scores (tokens with exact ties are skipped, where
    torch's order is unspecified)."""
    for order in (0, 1):
        w = synth.make_split("t", 79, 256, 64, 64, 8, 3, order=order)
        r = oracle.route(w)
        Hs = torch.from_numpy(r["H"]).double()
        vals, idx = torch.topk(Hs, w.k, dim=1)
        ok = r["min_gap"] > 0
        assert np.array_equal(idx.numpy()[ok], r["topk_idx"][ok])
        if order == 0:
            ref = torch.softmax(vals, dim=1).numpy()
        else:
            ref = torch.gather(torch.softmax(Hs, dim=1), 1, idx).numpy()
        np.testing.assert_allclose(r["topk_w"][ok], ref[ok], rtol=1e-14, atol=1e-16)


def test_expert_rows_against_torch_ffn():
    """One expert = down(SiLU(gate x) * up x), torch float64 matmuls."""
    w = synth.make_independent("t", 80, 10, 96, 40, 3, 2, act="f32", wt="f32")
    tokens = np.arange(10)
    for e in range(3):
        h, E = oracle.expert_rows(w, e, tokens, want_h=True, h_round=oracle.H_EXACT)
        x = torch.from_numpy(w.x).double()
        g = x @ torch.from_numpy(w.Wgate[e]).double().T
        u = x @ torch.from_numpy(w.Wup[e]).double().T
        hr = torch.nn.functional.silu(g) * u
        Er = hr @ torch.from_numpy(w.Wdown[e]).double().T
        np.testing.assert_allclose(h, hr.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(E, Er.numpy(), rtol=1e-12, atol=1e-14)


def test_h_rounding_modes():
    """bf16 mode rounds h to bf16 (torch's fp32->bf16 agrees on fp32-exact
    values), fp32 mode to fp32."""
    w = synth.make_independent("t", 81, 6, 64, 32, 2, 1, act="f32", wt="f32")
    t = np.arange(6)
    hx, _ = oracle.expert_rows(w, 1, t, want_h=True, h_round=oracle.H_EXACT)
    h32, _ = oracle.expert_rows(w, 1, t, want_h=True, h_round=oracle.H_F32)
    hb, _ = oracle.expert_rows(w, 1, t, want_h=True, h_round=oracle.H_BF16)
    assert np.array_equal(h32, hx.astype(np.float32).astype(np.float64))
    lib = oracle.load()
    assert np.array_equal(hb, np.vectorize(lib.brute_round_bf16)(hx))
    assert np.abs(hb - hx).max() <= np.abs(hx).max() * 2 ** -8


def test_combine_rows_equals_combine_tokens():
    """The two-step combine (expert outputs of every slot first, then the
    gate-weighted sum for one capacity setting) gives the same bits as the
    one-step combine, with and without drops, in both orders."""
    for order, cap in ((synth.MIXTRAL, -1), (synth.MIXTRAL, 3), (synth.ST, 2), (synth.MIXTRAL, 0)):
        w = synth.make_independent("rows", 40 + cap, 24, 32, 16, 6, 3, act="f32", wt="f32", order=order,
                                   capacity=cap, out_scale=2.0)
        r = oracle.route(w)
        cap_ = oracle.capacity(w, r["topk_idx"])
        toks = np.array([0, 3, 5, 11, 23], np.int64)
        E = oracle.assignment_outputs(w, r["topk_idx"], toks)
        a64, a32 = oracle.combine_tokens(w, r["topk_idx"], r["topk_w"], cap_["slot"], toks)
        b64, b32 = oracle.combine_rows(w, r["topk_w"], cap_["slot"], E, toks)
        assert np.array_equal(a64, b64) and np.array_equal(a32, b32)
        if cap == 0:
            assert np.all(b64 == 0.0)


def _token(w, t):
    """Token t of w as a one-token workload (same weights and draws)."""
    return synth.Workload(w.name, 1, w.H, w.F, w.N, w.k, w.capacity, w.order, w.noisy, False, w.out_scale, w.act,
                          w.wt, np.ascontiguousarray(w.x[t:t + 1]), w.Wg, w.Wn,
                          np.ascontiguousarray(w.eps[t:t + 1]), w.Wgate, w.Wup, w.Wdown)


def test_smooth_load_against_monte_carlo():
    """P(x, i) is the probability that expert i lands in the top k when only
    its own normal draw is taken again (the other experts keep their scores):
    estimated here by sampling that draw, with the rank taken over the whole
    score vector, it must agree with the oracle within 5 standard errors."""
    w = synth.make_independent("smooth", 70, 6, 64, 8, 6, 2, act="f32", wt="f32", noisy=True, wsig=0.3)
    rng = np.random.default_rng(7)
    M = 200_000
    for t in range(w.T):
        wt = _token(w, t)
        r = oracle.route(wt)
        P = oracle.smooth_load(wt)
        n = torch.from_numpy(wt.x).double() @ torch.from_numpy(wt.Wn).double()
        sp = torch.nn.functional.softplus(n)[0].numpy()
        Hs = r["H"][0].astype(np.float64)
        for i in range(w.N):
            z = rng.standard_normal(M)
            hi = float(r["logits"][0, i]) + z * sp[i]
            others = np.delete(Hs, i)
            rank = (others[None, :] > hi[:, None]).sum(axis=1)
            frac = float(np.mean(rank < w.k))
            se = np.sqrt(max(P[i] * (1 - P[i]), 1e-12) / M)
            assert abs(frac - P[i]) <= 5 * se + 1e-9, (t, i, frac, P[i])


def test_smooth_load_limits():
    """k = N keeps every expert whatever its draw: each P = 1, load = T. With
    the noise scale driven to ~0 (Softplus of a very negative noise logit),
    P becomes the indicator that the clean logit beats the others' k-th
    score, so the smooth load equals the hard load of the clean gate."""
    w = synth.make_independent("smooth_kn", 71, 9, 32, 8, 4, 4, act="f32", wt="f32", noisy=True)
    np.testing.assert_array_equal(oracle.smooth_load(w), np.full(4, 9.0))
    w = synth.make_independent("smooth_lim", 72, 40, 32, 8, 6, 2, act="f32", wt="f32", noisy=True)
    w.x = np.abs(w.x) + 0.5                       # every x.W_noise below -40 with W_noise = -1
    w.Wn = np.full_like(w.Wn, -1.0)
    w.Wg = synth.normal_f32(72, 99, w.Wg.shape, 1.0)
    r = oracle.route(w)
    assert np.all(r["min_gap"] > 1e-9)            # far above the noise scale of ~1e-18
    hard = np.bincount(r["topk_idx"].ravel(), minlength=w.N).astype(np.float64)
    np.testing.assert_allclose(oracle.smooth_load(w), hard, atol=1e-12)


def test_smooth_load_needs_the_noisy_gate():
    w = synth.make_independent("smooth_clean", 73, 4, 16, 8, 4, 2, act="f32", wt="f32")
    with pytest.raises(ValueError):
        oracle.smooth_load(w)
