"""The oracle's backward of the layer, pinned to things other than itself.

B1  central finite differences of L = <dy, y> + lambda * balance in exact
    arithmetic (h not rounded), for every input and weight of a tiny noisy
    layer with a capacity that drops slots, in both gate orders;
B2  upcycled identical experts (Mixtral, s = 1, dropless) make y = FFN(x)
    for any routing, so the router's gradient is exactly zero and the expert
    gradients sum to the dense FFN's, taken here by torch autograd in
    float64;
B3  the split layer with a zero router, k = N, s = N is the dense FFN:
    dx and the stacked expert gradients equal torch autograd's;
B4  the bf16 mode rounds only the matrix-core operands (dE, dg, du): it stays
    within bf16 rounding of the exact mode.
"""
import numpy as np
import torch

import oracle
import synth


def _loss(w, dy, lam):
    out = oracle.forward(w, h_round=oracle.H_EXACT)
    r = oracle.route(w)
    bal = oracle.stats(w, r)["balance"] if lam else 0.0
    return float(np.sum(dy.astype(np.float64) * out["y64"])) + lam * bal, out


def _tiny(order, seed):
    w = synth.make_independent("bwd", seed, 6, 8, 4, 4, 2, act="f32", wt="f32", order=order, noisy=True,
                               out_scale=2.0, capacity=2, wsig=0.5)
    w.want_stats = True
    return w


def _fd_check(w, dy, lam, names, delta=2.0 ** -9, tol=2e-3):
    g = oracle.backward(w, dy, lam, h_round=oracle.H_EXACT)
    base_idx = oracle.route(w)["topk_idx"]
    key = {"x": "dx", "Wg": "dWg", "Wn": "dWn", "Wgate": "dWgate", "Wup": "dWup", "Wdown": "dWdown"}
    for name in names:
        arr = getattr(w, name)
        fd = np.zeros(arr.shape)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = np.float32(keep + delta)
            lp, _ = _loss(w, dy, lam)
            assert np.array_equal(oracle.route(w)["topk_idx"], base_idx), "routing flipped under the step"
            flat[i] = np.float32(keep - delta)
            lm, _ = _loss(w, dy, lam)
            flat[i] = keep
            fd.reshape(-1)[i] = (lp - lm) / (2 * delta)
        got = g[key[name]]
        err = np.linalg.norm(got - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < tol, (name, err)
        assert np.linalg.norm(fd) > 0


def test_B1_finite_differences_mixtral_and_st():
    for order, seed in ((synth.MIXTRAL, 90), (synth.ST, 91)):
        w = _tiny(order, seed)
        r = oracle.route(w)
        assert np.all(r["min_gap"] > 0.02), "pick inputs without near ties"
        cap = oracle.capacity(w, r["topk_idx"])
        assert np.any(cap["slot"] < 0), "the capacity must drop a slot"
        dy = synth.normal_f32(seed, 30, (w.T, w.H), 1.0)
        _fd_check(w, dy, 0.7, ["x", "Wg", "Wn", "Wgate", "Wup", "Wdown"])


def test_B1_finite_differences_clean_gate():
    w = synth.make_independent("bwd_clean", 92, 5, 8, 4, 3, 2, act="f32", wt="f32", out_scale=1.5, wsig=0.5)
    assert np.all(oracle.route(w)["min_gap"] > 0.02)
    dy = synth.normal_f32(92, 30, (w.T, w.H), 1.0)
    _fd_check(w, dy, 0.0, ["x", "Wg", "Wgate", "Wup", "Wdown"])
    g = oracle.backward(w, dy, 0.0, h_round=oracle.H_EXACT)
    assert np.all(g["dWn"] == 0.0)


def _dense_grads(x, Wg_d, Wu_d, Wd_d, dy):
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_()
    a = torch.from_numpy(Wg_d.astype(np.float64)).requires_grad_()
    b = torch.from_numpy(Wu_d.astype(np.float64)).requires_grad_()
    d = torch.from_numpy(Wd_d.astype(np.float64)).requires_grad_()
    y = (torch.nn.functional.silu(xt @ a.T) * (xt @ b.T)) @ d.T
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return xt.grad.numpy(), a.grad.numpy(), b.grad.numpy(), d.grad.numpy()


def test_B2_upcycled_identical_experts():
    w = synth.make_upcycled("bwd_up", 93, 12, 16, 8, 4, 2, perturb=0.0, keep_base=True)
    w.x = synth.f32_to_bf16(synth.bf16_to_f32(w.x))
    dy = synth.normal_f32(93, 30, (w.T, w.H), 1.0)
    g = oracle.backward(w, dy, 0.0, h_round=oracle.H_EXACT)
    assert np.abs(g["dWg"]).max() < 1e-12
    Wg_d, Wu_d, Wd_d = (synth.bf16_to_f32(w.Wgate[0]), synth.bf16_to_f32(w.Wup[0]), synth.bf16_to_f32(w.Wdown[0]))
    dx, da, db, dd = _dense_grads(synth.bf16_to_f32(w.x), Wg_d, Wu_d, Wd_d, dy)
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWgate"].sum(axis=0), da, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWup"].sum(axis=0), db, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWdown"].sum(axis=0), dd, rtol=1e-10, atol=1e-12)


def test_B3_zero_router_all_experts_is_the_dense_ffn():
    N = 4
    w = synth.make_split("bwd_split", 94, 10, 16, N * 4, N, N, act="f32", wt="f32", out_scale=float(N))
    w.Wg = np.zeros_like(w.Wg)
    dy = synth.normal_f32(94, 30, (w.T, w.H), 1.0)
    g = oracle.backward(w, dy, 0.0, h_round=oracle.H_EXACT)
    Wg_d, Wu_d, Wd_d = w.meta["dense"]
    dx, da, db, dd = _dense_grads(w.x, Wg_d, Wu_d, Wd_d, dy)
    perm = w.meta["perm"].reshape(N, -1)
    np.testing.assert_allclose(g["dx"], dx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWgate"], da[perm], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWup"], db[perm], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dWdown"], np.transpose(dd[:, perm], (1, 0, 2)), rtol=1e-10, atol=1e-12)


def test_B4_bf16_mode_rounds_only_the_operands():
    w = synth.make_independent("bwd_bf", 95, 40, 64, 32, 8, 2, noisy=True, out_scale=4.0)
    dy = synth.normal_f32(95, 30, (w.T, w.H), 1.0)
    a = oracle.backward(w, dy, 0.5)
    b = oracle.backward(w, dy, 0.5, h_round=oracle.H_EXACT)
    for key in a:
        if key == "dWn" and not w.noisy:
            continue
        err = np.linalg.norm(a[key] - b[key]) / np.linalg.norm(b[key])
        assert 1e-5 < err < 2e-2, (key, err)


def test_B5_thread_count_does_not_change_a_bit():
    """Every sum in the backward keeps a fixed order (an expert's rows in
    token order, a token's slots in slot order, tokens in order), so the
    threaded run gives the single-threaded run's bits."""
    w = synth.make_independent("bwd_thr", 96, 60, 64, 32, 6, 2, noisy=True, order=synth.ST, capacity=18,
                               out_scale=3.0)
    dy = synth.normal_f32(96, 30, (w.T, w.H), 1.0)
    a = oracle.backward(w, dy, 0.2, nthreads=1)
    b = oracle.backward(w, dy, 0.2, nthreads=5)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
