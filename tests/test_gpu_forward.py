"""moe_forward (the whole layer in one call) against the oracle.

Every test compares every output element (all tokens) with the oracle, on
small shapes of every workload family, on a mid-sized layer whose expert
kernel runs about three rounds of tiles per workgroup, and on the five named
workloads at full size in the same launch configuration as the benchmark.
The C4 capacity variants share one oracle pass over the experts (every slot
of every token), combined per capacity setting."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_forward, check_smooth_load, log, oracle_threads, run_forward, upload

pytestmark = pytest.mark.gpu

SMALL = {
    "split_bf16_s4": lambda: synth.make_split("split_bf16_s4", 21, 333, 512, 8 * 48, 8, 2, out_scale=4.0),
    "split_noisy_stats": lambda: synth.make_split("split_noisy", 22, 400, 512, 16 * 24, 16, 4, noisy=True,
                                                  want_stats=True, out_scale=4.0),
    "upcycled_cf1": lambda: synth.make_upcycled("up_cf1", 23, 512, 256, 128, 8, 2,
                                                capacity=synth.capacity_from_cf(512, 8, 2, 1.0)),
    "upcycled_cf4": lambda: synth.make_upcycled("up_cf4", 24, 512, 256, 128, 8, 2,
                                                capacity=synth.capacity_from_cf(512, 8, 2, 4.0)),
    "upcycled_dropless": lambda: synth.make_upcycled("up_dl", 25, 300, 256, 192, 8, 2),
    "decode_skewed": lambda: synth.apply_skew(synth.make_independent("dec", 26, 64, 512, 1024, 8, 2), n_pref=32),
    # decode-shaped tiles with K tails inside a K step in both GEMMs (H 1032,
    # F 1376), a ragged last column tile, and the down projection split over K
    "decode_k_tails": lambda: synth.make_independent("deck", 39, 30, 1032, 1376, 8, 2),
    "fp32_split": lambda: synth.make_split("fp32", 27, 200, 128, 8 * 40, 8, 2, act="f32", wt="f32"),
    "st_order": lambda: synth.make_split("st", 28, 150, 256, 8 * 32, 8, 2, order=synth.ST),
    "bf16_f_not_mult8": lambda: synth.make_independent("f86", 29, 100, 256, 86, 8, 2, out_scale=4.0),
    "one_expert": lambda: synth.make_independent("n1", 30, 70, 128, 64, 1, 1),
    "k_equals_n": lambda: synth.make_independent("keqn", 31, 90, 128, 64, 4, 4),
    "one_token": lambda: synth.make_independent("t1", 32, 1, 256, 64, 8, 2),
    "capacity_zero": lambda: synth.make_independent("c0", 33, 50, 128, 32, 8, 2, capacity=0),
    "n64_k8": lambda: synth.make_independent("n64", 34, 200, 256, 64, 64, 8),
    # the persistent expert kernel at the edges of its per-lane expert scans:
    # 64 experts (one per lane) and a single expert
    "fused_n64_k4": lambda: synth.make_independent("fn64", 37, 1024, 256, 64, 64, 4),
    "fused_n1": lambda: synth.make_independent("fn1", 38, 600, 256, 136, 1, 1),
    # prefill-sized, with three quarters of the tokens steered to expert 0: one
    # expert owns many row blocks of the persistent expert kernel
    "prefill_skewed": lambda: synth.apply_skew(synth.make_independent("pskew", 36, 2048, 512, 256, 8, 2),
                                               n_pref=1536),
    # about 780 tiles of the persistent expert kernel (row blocks x (12 gate/up
    # + 8 down tiles)) over 256 workgroups: about three rounds, so workgroups
    # reserve a next ticket, issue its first stage into the free stage buffer
    # (gate/up and down kinds), and down tiles wait on gate/up tiles of later
    # rounds; half the tokens are steered to expert 0, which owns nine row
    # blocks, and every expert ends in a partly filled row block
    "multi_round": lambda: synth.apply_skew(synth.make_independent("mround", 42, 4000, 2048, 1536, 8, 2,
                                                                   out_scale=4.0), n_pref=2000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    w = SMALL[name]()
    g, ora, cap = check_forward(w)
    if w.capacity == 0:
        assert np.all(g["y"] == 0.0)
    if w.want_stats:
        st = oracle.stats(w, ora)
        np.testing.assert_allclose(g["importance"], st["importance"], rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(g["P"], st["P"], rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(g["balance"][0], st["balance"], rtol=1e-5)
        if w.noisy:
            check_smooth_load(g["smooth_load"], w, name)


def test_forward_bf16_output_within_one_ulp():
    w = SMALL["split_bf16_s4"]()
    g = run_forward(w, out="bf16")
    ora = oracle.forward(w)
    ref = ora["y"].astype(np.float64)
    ulp = np.spacing(np.abs(synth.bf16_to_f32(synth.f32_to_bf16(ora["y"])))).astype(np.float64) * 65536.0
    # one bf16 step plus the fp32 error of the layer before rounding
    assert np.all(np.abs(g["y"] - ref) <= ulp + 2e-2)
    assert np.mean(np.abs(g["y"] - ref) <= ulp) > 0.99


def test_forward_empty_batch():
    w = synth.make_independent("t0", 35, 0, 128, 64, 8, 2, want_stats=True)
    w.x = np.zeros((0, 128), np.uint16)
    w.eps = None
    g = run_forward(w)
    assert g["y"].shape == (0, 128)
    assert np.all(g["kept"] == 0) and np.all(g["load"] == 0)


def test_forward_is_deterministic():
    w = SMALL["split_noisy_stats"]()
    d = upload(w)
    a = run_forward(w, d=d)
    b = run_forward(w, d=d)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_forward_follows_the_callers_stream():
    """Every launch goes to the stream the caller makes current: on a side
    stream whose x is written only after a long matmul, the layer must read
    the new x (a launch on another stream would race ahead and see zeros)."""
    w = synth.make_split("strm", 41, 1200, 1024, 8 * 96, 8, 2, out_scale=4.0, want_stats=True)
    d = upload(w)
    ref = run_forward(w, d=d)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x2 = torch.zeros_like(d["x"])
        m = torch.randn(4096, 4096, device="cuda")
        for _ in range(8):
            m = torch.mm(m, m) * 1e-3  # keeps the side stream busy for a while
        x2.copy_(d["x"])
        got = run_forward(w, d=dict(d, x=x2))
    side.synchronize()
    for key in ref:
        assert np.array_equal(ref[key], got[key]), key
    del m


def test_full_C2_is_deterministic():
    """The expert GEMMs run as one persistent launch whose workgroups take
    tiles from a queue in whatever order they arrive; every output element is
    still computed by one tile in a fixed K order, so two runs agree bit for
    bit."""
    w = synth.c2()
    d = upload(w)
    a = run_forward(w, d=d)
    b = run_forward(w, d=d)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---- the five named workloads at full size, every token --------------------------

@functools.lru_cache(maxsize=1)
def _c4_base():
    """C4's inputs, the oracle's routing (the same for every capacity
    variant), and the oracle's expert output for every slot of every token."""
    w = synth.c4("dropless")
    ora = oracle.route(w)
    log(f"[C4] oracle experts for all {w.T * w.k} slots on {oracle_threads()} threads")
    E = oracle.assignment_outputs(w, ora["topk_idx"], nthreads=oracle_threads())
    return w, ora, E


def _c4(variant):
    w, ora, E = _c4_base()
    cap = {"cf4": synth.capacity_from_cf(w.T, 8, 2, 4.0), "cf1": synth.capacity_from_cf(w.T, 8, 2, 1.0),
           "dropless": -1, "cf1_assign": synth.capacity_from_cf(w.T, 8, 2, 1.0, True)}[variant]
    v = synth.Workload(f"C4_{variant}", w.T, w.H, w.F, w.N, w.k, cap, w.order, False, False, 1.0, "bf16", "bf16",
                       w.x, w.Wg, None, None, w.Wgate, w.Wup, w.Wdown, dict(w.meta))
    return v, ora, E


def test_full_C1():
    check_forward(synth.c1())


def test_full_C2():
    check_forward(synth.c2())


def test_full_C3():
    w = synth.c3()
    g, ora, _ = check_forward(w)
    st = oracle.stats(w, ora)
    np.testing.assert_allclose(g["importance"], st["importance"], rtol=1e-5)
    np.testing.assert_allclose(g["P"], st["P"], rtol=1e-5)
    np.testing.assert_allclose(g["balance"][0], st["balance"], rtol=1e-5)
    check_smooth_load(g["smooth_load"], w, "C3")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("variant", ["cf4", "cf1", "dropless", "cf1_assign"])
def test_full_C4(variant):
    w, ora, E = _c4(variant)
    g, _, cap = check_forward(w, ora=ora, E=E)
    log(f"  kept per expert {g['kept'].tolist()} (capacity {w.capacity}); "
        f"{int(np.sum(cap['slot'] < 0))} slots dropped")
    if w.capacity >= 0:
        assert np.all(g["kept"] <= w.capacity)


def test_full_switch_top1():
    """Switch-style routing at the LLaMA-MoE-3.5B 2/8 layer shape: top-1,
    softmax over all experts then top-k (ST order), dropless."""
    w = synth.make_split("switch_top1", 1006, 4096, 4096, 11008, 8, 1, order=synth.ST, out_scale=1.0)
    g, ora, _ = check_forward(w)
    assert np.all(g["topk_w"][:, 0] < 1.0)  # ST weights are not renormalised


def test_full_C5():
    w = synth.c5()
    g, _, _ = check_forward(w)
    frac = float(np.mean(g["topk_idx"][:, 0] == 0))
    log(f"  C5 top-1 fraction on expert 0: {frac:.3f}; rows per expert {g['kept'].tolist()}")
    assert frac >= 0.5
