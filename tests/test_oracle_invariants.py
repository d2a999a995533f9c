"""Invariants the method fixes, checked on the oracle.

I1  gate weights sum to 1 (Mixtral order) / to the top-k softmax mass (ST).
I2a the experts of a non-overlapping split sum to the dense FFN.
I2b zero router, k = N, s = N: the layer reproduces the dense FFN.
I3  identical (upcycled) experts reproduce the dense FFN for any router;
    with capacity, y_t = (sum of kept w) * FFN(x_t).
I4  kept_i = min(load_i, C) <= C and sum kept = number of rows.
I5  slot and row_token are inverse; rows of an expert are in token order.
I6  dropless equals a capacity >= T; capacity 0 gives y = 0.
I7  eps = 0 makes the noisy gate equal the clean one.
I8  stats closed form at a zero router.
I9  k = 1 Mixtral gives w = 1; all-equal scores give w = 1/k on 0..k-1.
I10 dropless outputs are equivariant under token permutation.
I11 relabelling the experts leaves y unchanged (no score ties).
I12 a NaN router score ranks as -inf: the layer equals the same layer
    without that expert (reading of the pages' silence on non-numbers).
"""
import numpy as np
import torch

import oracle
import synth


def dense_ffn(x, Wg_d, Wu_d, Wd_d):
    x = torch.from_numpy(x).double()
    g = x @ torch.from_numpy(Wg_d).double().T
    u = x @ torch.from_numpy(Wu_d).double().T
    return ((torch.nn.functional.silu(g) * u) @ torch.from_numpy(Wd_d).double().T).numpy()


def f32_split(seed, T=24, H=32, Ftot=96, N=6, k=2, **kw):
    return synth.make_split("inv", seed, T, H, Ftot, N, k, act="f32", wt="f32", **kw)


def test_I1_gate_sums():
    for order in (0, 1):
        w = f32_split(1, order=order, N=8, k=3)
        r = oracle.route(w)
        s = r["topk_w"].sum(axis=1)
        if order == 0:
            np.testing.assert_allclose(s, 1.0, atol=1e-14)
        else:
            p = torch.softmax(torch.from_numpy(r["H"]).double(), dim=1).numpy()
            top = np.sort(p, axis=1)[:, ::-1][:, :3].sum(axis=1)
            np.testing.assert_allclose(s, top, atol=1e-14)
            assert np.all(s <= 1.0 + 1e-15)


def test_I2a_split_identity():
    w = f32_split(2)
    Wg_d, Wu_d, Wd_d = w.meta["dense"]
    tokens = np.arange(w.T)
    tot = sum(oracle.expert_rows(w, e, tokens, h_round=oracle.H_EXACT) for e in range(w.N))
    ref = dense_ffn(w.x, Wg_d, Wu_d, Wd_d)
    np.testing.assert_allclose(tot, ref, rtol=1e-12, atol=1e-13)


def test_I2b_zero_router_all_experts_is_dense():
    w = f32_split(3, k=6, N=6, out_scale=6.0)
    w.Wg = np.zeros_like(w.Wg)
    out = oracle.forward(w, h_round=oracle.H_EXACT)
    assert np.all(out["topk_w"] == 1.0 / 6.0)
    ref = dense_ffn(w.x, *w.meta["dense"])
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-13)
    # fp32 h rounding stays within fp32 relative accuracy
    out32 = oracle.forward(w, h_round=oracle.H_F32)
    np.testing.assert_allclose(out32["y64"], ref, rtol=1e-5, atol=1e-6)


def _upcycled_f32(seed, T=20, H=16, F=12, N=4, k=2, capacity=-1):
    base = synth.make_independent("up", seed, T, H, F, 1, 1, act="f32", wt="f32")
    w = synth.make_independent("up", seed, T, H, F, N, k, act="f32", wt="f32", capacity=capacity)
    w.Wgate = np.ascontiguousarray(np.repeat(base.Wgate, N, axis=0))
    w.Wup = np.ascontiguousarray(np.repeat(base.Wup, N, axis=0))
    w.Wdown = np.ascontiguousarray(np.repeat(base.Wdown, N, axis=0))
    w.Wg = synth.normal_f32(seed, 99, (H, N), 1.0)  # any router
    return w, base


def test_I3_upcycled_identical_experts_reproduce_dense():
    w, base = _upcycled_f32(4)
    out = oracle.forward(w, h_round=oracle.H_EXACT)
    ref = dense_ffn(w.x, base.Wgate[0], base.Wup[0], base.Wdown[0])
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-13)


def test_I3_upcycled_with_capacity_scales_by_kept_weight():
    w, base = _upcycled_f32(5, T=40, capacity=6)
    out = oracle.forward(w, h_round=oracle.H_EXACT)
    ref = dense_ffn(w.x, base.Wgate[0], base.Wup[0], base.Wdown[0])
    kept_w = np.where(out["slot"] >= 0, out["topk_w"], 0.0).sum(axis=1)
    assert (kept_w < 1 - 1e-9).any()  # some assignments were dropped
    np.testing.assert_allclose(out["y64"], kept_w[:, None] * ref, rtol=1e-12, atol=1e-13)


def test_I4_I5_capacity_and_permutation_structure():
    for cap in (-1, 0, 1, 5, 9, 1000):
        w = f32_split(6, T=60, N=8, k=3, capacity=cap)
        r = oracle.route(w)
        c = oracle.capacity(w, r["topk_idx"])
        load = np.bincount(r["topk_idx"].ravel(), minlength=w.N)
        assert np.array_equal(c["counts"], load)
        C = cap if cap >= 0 else 10 ** 9
        assert np.array_equal(c["kept"], np.minimum(load, C))
        assert np.all(c["kept"] <= C)
        A = int(c["kept"].sum())
        assert c["offsets"][-1] == A
        assert np.array_equal(np.diff(c["offsets"]), c["kept"])
        rows = c["slot"][c["slot"] >= 0]
        assert np.array_equal(np.sort(rows), np.arange(A))
        for t in range(w.T):
            for j in range(w.k):
                s = c["slot"][t, j]
                if s >= 0:
                    assert c["row_token"][s] == t
                    e = r["topk_idx"][t, j]
                    assert c["offsets"][e] <= s < c["offsets"][e + 1]
        assert np.all(c["row_token"][A:] == -1)
        for e in range(w.N):
            seg = c["row_token"][c["offsets"][e]:c["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)
            # the kept tokens are the first ones routed to e, in token order
            routed = np.nonzero((r["topk_idx"] == e).any(axis=1))[0]
            assert np.array_equal(seg, routed[:len(seg)])


def test_I6_dropless_equals_large_capacity_and_zero_capacity_is_zero():
    w = f32_split(7)
    a = oracle.forward(w)
    w.capacity = w.T
    b = oracle.forward(w)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["slot"], b["slot"])
    w.capacity = 0
    z = oracle.forward(w)
    assert np.all(z["y"] == 0) and np.all(z["slot"] == -1)


def test_I7_zero_noise_equals_clean_gate():
    w = f32_split(8, noisy=True, N=8, k=2)
    w.eps = np.zeros_like(w.eps)
    a = oracle.forward(w)
    w.noisy = False
    b = oracle.forward(w)
    assert np.array_equal(a["H"], b["H"]) and np.array_equal(a["y"], b["y"])


def test_I8_stats_closed_form_at_zero_router():
    for N, k in ((8, 2), (16, 4), (5, 5)):
        w = f32_split(9, N=N, k=k, Ftot=N * 4)
        w.Wg = np.zeros_like(w.Wg)
        r = oracle.route(w)
        st = oracle.stats(w, r)
        np.testing.assert_allclose(st["P"], 1.0 / N, atol=1e-15)
        f = np.where(np.arange(N) < k, 1.0 / k, 0.0)
        np.testing.assert_allclose(st["f"], f, atol=1e-15)
        assert abs(st["balance"] - 1.0 / N) < 1e-15
        assert st["load"].sum() == w.T * k
        assert abs(st["importance"].sum() - w.T) < 1e-12
        # the code example's variant: importance shares (1/k on the first k)
        # times the uniform P, times N, with its 1e-6 guard on the total
        assert abs(st["balance_code"] - w.T / (w.T + 1e-6)) < 1e-14


def test_I8b_code_balance_hand_case():
    """One token, two experts, ST order, top-1, logits (l, 0) with
    l = fl32(ln 3): softmax = (p, 1 - p), p = 1 / (1 + e^-l), so expert 0 is
    kept with weight p; importance = (p, 0), P = (p, 1 - p), f = (1, 0).
    balance = p; the code example's variant = N * (p / (p + 1e-6)) * p."""
    l = float(np.float32(np.log(3.0)))
    w = synth.Workload("bal", 1, 1, 1, 2, 1, -1, synth.ST, False, True, 1.0, "f32", "f32",
                       x=np.ones((1, 1), np.float32), Wg=np.array([[l, 0.0]], np.float32))
    r = oracle.route(w)
    st = oracle.stats(w, r)
    p = 1.0 / (1.0 + np.exp(-l))
    assert r["topk_idx"].tolist() == [[0]]
    assert abs(r["topk_w"][0, 0] - p) < 1e-15
    assert abs(st["balance"] - p) < 1e-15
    assert abs(st["balance_code"] - 2.0 * (p / (p + 1e-6)) * p) < 1e-15


def test_I9_k1_and_equal_scores():
    w = f32_split(10, k=1)
    r = oracle.route(w)
    assert np.all(r["topk_w"] == 1.0)
    w = f32_split(11, k=4, N=6, Ftot=24)
    w.Wg = np.zeros_like(w.Wg)
    r = oracle.route(w)
    assert np.all(r["topk_idx"] == np.arange(4)) and np.all(r["topk_w"] == 0.25)


def test_I10_token_permutation_equivariance():
    w = f32_split(12, T=32)
    a = oracle.forward(w)
    p = np.random.default_rng(0).permutation(w.T)
    w.x = np.ascontiguousarray(w.x[p])
    b = oracle.forward(w)
    assert np.array_equal(a["y"][p], b["y"])
    assert np.array_equal(a["topk_idx"][p], b["topk_idx"])


def test_I11_expert_relabelling_invariance():
    w = f32_split(13, T=32, N=6, k=2)
    a = oracle.forward(w)
    assert np.all(a["min_gap"] > 0)
    q = np.random.default_rng(1).permutation(w.N)
    w.Wg = np.ascontiguousarray(w.Wg[:, q])
    w.Wgate = np.ascontiguousarray(w.Wgate[q])
    w.Wup = np.ascontiguousarray(w.Wup[q])
    w.Wdown = np.ascontiguousarray(w.Wdown[q])
    b = oracle.forward(w)
    np.testing.assert_allclose(a["y64"], b["y64"], rtol=1e-13, atol=1e-14)
    assert np.array_equal(q[b["topk_idx"]], a["topk_idx"])


def test_empty_batch():
    w = f32_split(14, T=0)
    w.x = np.zeros((0, w.H), np.float32)
    out = oracle.forward(w)
    assert out["y"].shape == (0, w.H)
    assert np.all(out["counts"] == 0) and np.all(out["offsets"] == 0)


def test_I12_nan_score_ranks_below_every_number():
    """A NaN router column (expert 2) is never chosen while k < N, and the
    routing and output equal those of the same layer without expert 2, in
    both orders; with k = N it is kept last, with weight 0."""
    for order in (synth.MIXTRAL, synth.ST):
        w = f32_split(15, T=20, N=5, k=2, Ftot=5 * 8, order=order)
        drop = 2
        keep = [e for e in range(w.N) if e != drop]
        v = synth.Workload("nan_ref", w.T, w.H, w.F, w.N - 1, w.k, -1, order, False, False, 1.0, "f32", "f32",
                           x=w.x, Wg=np.ascontiguousarray(w.Wg[:, keep]),
                           Wgate=np.ascontiguousarray(w.Wgate[keep]), Wup=np.ascontiguousarray(w.Wup[keep]),
                           Wdown=np.ascontiguousarray(w.Wdown[keep]))
        w.Wg = w.Wg.copy()
        w.Wg[:, drop] = np.nan
        a = oracle.forward(w)
        b = oracle.forward(v)
        assert np.array_equal(np.array(keep)[b["topk_idx"]], a["topk_idx"])
        np.testing.assert_array_equal(a["topk_w"], b["topk_w"])
        np.testing.assert_array_equal(a["y64"], b["y64"])
        assert np.all(np.isneginf(a["H"][:, drop]))
    w = f32_split(16, T=10, N=3, k=3, Ftot=3 * 8)
    w.Wg = w.Wg.copy()
    w.Wg[:, 1] = np.nan
    a = oracle.route(w)
    assert np.all(a["topk_idx"][:, 2] == 1) and np.all(a["topk_w"][:, 2] == 0.0)
    np.testing.assert_allclose(a["topk_w"].sum(axis=1), 1.0, rtol=1e-15)


def test_I13_residual_layer_reduces_to_the_dense_ffn():
    """Shared slice + routed experts of one dense FFN (the Inter / residual
    mode): with a zero router (every gate 1/N), k = N and s = N, the routed
    experts sum to the rest of the FFN, so the layer is the dense FFN."""
    w = synth.make_residual("res", 17, 12, 32, 8 * 6 + 16, 16, 6, 6, act="f32", wt="f32", out_scale=6.0)
    w.Wg = np.zeros_like(w.Wg)
    out = oracle.residual_forward(w, h_round=oracle.H_EXACT)
    Wg_d, Wu_d, Wd_d = w.meta["dense"]
    np.testing.assert_allclose(out["y64"], dense_ffn(w.x, Wg_d, Wu_d, Wd_d), rtol=1e-12, atol=1e-13)


def test_I14_residual_layer_with_every_slot_dropped_is_the_shared_slice():
    """Capacity 0 drops every routed slot: the output is exactly the shared
    slice's FFN, which equals the dense FFN restricted to those neurons."""
    w = synth.make_residual("res0", 18, 10, 32, 4 * 8 + 8, 8, 4, 2, act="f32", wt="f32", capacity=0, out_scale=2.0)
    out = oracle.residual_forward(w, h_round=oracle.H_EXACT)
    assert np.array_equal(out["y64"], out["R"])
    Wg_d, Wu_d, Wd_d = w.meta["dense"]
    sh = w.meta["perm"][:8]
    np.testing.assert_allclose(out["y64"], dense_ffn(w.x, Wg_d[sh], Wu_d[sh], Wd_d[:, sh]), rtol=1e-12, atol=1e-13)


def test_I15_residual_adds_the_shared_slice_to_the_plain_layer():
    """The routed part is the plain layer of the same experts: y - R equals
    the one-step oracle's output (same routing, slots and scale)."""
    w = synth.make_residual("res_r", 19, 16, 32, 4 * 8 + 8, 8, 4, 2, act="f32", wt="f32", capacity=5,
                            out_scale=2.0)
    out = oracle.residual_forward(w)
    plain = oracle.forward(w)
    np.testing.assert_allclose(out["y64"] - out["R"], plain["y64"], rtol=1e-12, atol=1e-13)
    assert np.any(out["slot"] < 0) and np.any(np.abs(out["R"]) > 0)


def test_I16_inner_sharing_expert_is_shared_plus_own_neurons():
    """Inner mode: an expert holding the shared neurons and its own is, in
    exact arithmetic, the shared slice's FFN plus its own slice's FFN."""
    w = synth.make_inner_shared("inner", 20, 8, 32, 4 * 8 + 8, 8, 4, 2, act="f32", wt="f32")
    r = w.meta["residual"]
    toks = np.arange(w.T)
    for e in range(w.N):
        got = oracle.expert_rows(w, e, toks, h_round=oracle.H_EXACT)
        want = (oracle.expert_rows(oracle.shared_slice(r), 0, toks, h_round=oracle.H_EXACT)
                + oracle.expert_rows(r, e, toks, h_round=oracle.H_EXACT))
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
