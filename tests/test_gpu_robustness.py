"""Inputs and conditions outside the normal path, through the C ABI: NaN
router scores, expert indices outside [0, N) handed to moe_permute, and the
expert kernel's bounded wait giving up (forced from the host). Every kernel
still ends normally; the guard bands around each workspace and output (see
gpu_util) catch any write past a buffer."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import cfg_of, check_forward, dev, guarded_empty, host, log, run_forward, upload, workspace
from sparse_mixture_experts_05_amd import abi

pytestmark = pytest.mark.gpu


def _with_nan_column(w, col):
    w.Wg = w.Wg.copy()
    w.Wg[:, col] = np.nan
    return w


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("order", [synth.MIXTRAL, synth.ST])
def test_nan_router_column_is_never_chosen(act, order):
    """One NaN column of W_g gives expert 3 a NaN score for every token; it
    ranks as -inf, so routing and output equal the oracle's (which takes the
    same reading) and the expert gets no rows."""
    w = _with_nan_column(synth.make_independent(f"nan_{act}_{order}", 51, 700, 512, 256, 8, 2, act=act, wt=act,
                                                order=order, out_scale=4.0), 3)
    g, ora, cap = check_forward(w)
    assert not np.any(g["topk_idx"] == 3)
    assert g["kept"][3] == 0 and int(g["kept"].sum()) == w.T * w.k


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_all_nan_router_keeps_exactly_k(act):
    """Every score NaN: every expert ties at -inf, so the first k experts are
    kept (ties to the lower index) and the row count stays T*k."""
    w = synth.make_independent(f"allnan_{act}", 52, 300, 256, 128, 8, 2, act=act, wt=act)
    w.Wg = np.full_like(w.Wg, np.nan)
    g = run_forward(w)
    assert np.all(g["topk_idx"] == np.arange(w.k))
    assert int(g["kept"].sum()) == w.T * w.k and int(g["load"].sum()) == w.T * w.k
    ora = oracle.route(w)
    assert np.array_equal(ora["topk_idx"], g["topk_idx"])


def test_permute_drops_indices_outside_the_experts():
    """moe_permute takes topk_idx from the caller: an index outside [0, N)
    is dropped (slot -1) and counts nowhere; the valid slots keep their
    first-come order per expert."""
    T, H, N, k = 500, 128, 8, 2
    rng = np.random.default_rng(5)
    idx = rng.integers(0, N, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx[bad] = rng.choice([-1, N, N + 7, -100000, 1 << 30], size=int(bad.sum()))
    cfg = abi.MoEConfig(T=T, H=H, F=64, N=N, k=k, capacity=40)
    counts = guarded_empty((N,), torch.int32)
    offsets = guarded_empty((N + 1,), torch.int32)
    slot = guarded_empty((T, k), torch.int32)
    row_token = guarded_empty((T * k,), torch.int32)
    x = dev(synth.normal_bf16(5, 0, (T, H)))
    x_perm = guarded_empty((T * k, H), torch.bfloat16)
    abi.moe_permute(cfg, x, dev(idx), counts, offsets, slot, row_token, x_perm, ws=workspace(cfg))
    torch.cuda.synchronize()
    counts, offsets, slot, row_token = host(counts), host(offsets), host(slot), host(row_token)
    valid = (idx >= 0) & (idx < N)
    want_counts = np.bincount(idx[valid], minlength=N)
    assert np.array_equal(counts, want_counts)
    kept = np.minimum(want_counts, 40)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(kept)]))
    assert np.all(slot[~valid] == -1)
    # first come, first kept, per expert, in token order
    seen = np.zeros(N, np.int64)
    for t in range(T):
        for j in range(k):
            if not valid[t, j]:
                continue
            e = idx[t, j]
            want = offsets[e] + seen[e] if seen[e] < 40 else -1
            seen[e] += 1
            assert slot[t, j] == want, (t, j)
            if want >= 0:
                assert row_token[want] == t
    assert np.all(row_token[offsets[-1]:] == -1)


def test_bounded_wait_failure_poisons_the_output():
    """Force every down tile's wait to give up (a count one above what the
    gate/up tiles reach, and a 64-poll limit): the tiles write NaN and the
    combine writes NaN over all of y. Then normal operation returns."""
    w = synth.make_split("waitfail", 53, 1500, 512, 8 * 256, 8, 2, out_scale=4.0)
    d = upload(w)
    ref = run_forward(w, d=d)
    assert np.all(np.isfinite(ref["y"]))
    try:
        abi.moe_debug_set_wait(64, 1)
        bad = run_forward(w, d=d)
    finally:
        abi.moe_debug_set_wait(0, 0)
    assert np.all(np.isnan(bad["y"])), "a failed wait must not pass as a result"
    assert np.array_equal(bad["topk_idx"], ref["topk_idx"])
    again = run_forward(w, d=d)
    for key in ref:
        assert np.array_equal(ref[key], again[key], equal_nan=False), key
    log("  bounded wait: forced failure gave an all-NaN y; the next call matches the first bit for bit")



def test_permute_repeated_expert_in_a_row_matches_the_oracle():
    """A caller's topk_idx may name one expert in two slots of a token: each
    entry is its own assignment, ranked in (token, slot) order, exactly as the
    oracle's sequential counters rank it."""
    T, H, N, k, C = 700, 64, 6, 3, 150
    rng = np.random.default_rng(6)
    idx = rng.integers(0, N, size=(T, k)).astype(np.int32)
    assert np.any(idx[:, 0] == idx[:, 1])
    w = synth.Workload("dup", T, H, 32, N, k, C, x=np.zeros((T, H), np.float32))
    ref = oracle.capacity(w, idx)
    cfg = abi.MoEConfig(T=T, H=H, F=32, N=N, k=k, capacity=C)
    counts = guarded_empty((N,), torch.int32)
    offsets = guarded_empty((N + 1,), torch.int32)
    slot = guarded_empty((T, k), torch.int32)
    row_token = guarded_empty((T * k,), torch.int32)
    abi.moe_permute(cfg, None, dev(idx), counts, offsets, slot, row_token, None, ws=workspace(cfg))
    torch.cuda.synchronize()
    assert np.array_equal(host(counts), ref["counts"])
    assert np.array_equal(host(offsets), ref["offsets"])
    assert np.array_equal(host(slot), ref["slot"])
    assert np.array_equal(host(row_token), ref["row_token"])
