"""The seeded input generator: reproducible, slice-stable, correctly
distributed, and the expert split is a partition of the dense FFN."""
import numpy as np
import torch

import synth


def test_reproducible_and_slice_stable():
    a = synth.normal_f32(5, 3, (1000,), 1.0)
    b = synth.normal_f32(5, 3, (1000,), 1.0)
    assert np.array_equal(a, b)
    c = synth.normal_f32(5, 3, (400,), 1.0, offset=600)
    assert np.array_equal(a[600:], c)
    d = synth.normal_f32(5, 4, (1000,), 1.0)
    assert not np.array_equal(a, d)
    e = synth.normal_f32(6, 3, (1000,), 1.0)
    assert not np.array_equal(a, e)


def test_normal_moments():
    z = synth.normal_f32(11, 0, (2_000_000,), 1.0).astype(np.float64)
    assert abs(z.mean()) < 3e-3
    assert abs(z.std() - 1.0) < 3e-3
    # fourth moment of a standard normal is 3
    assert abs((z ** 4).mean() - 3.0) < 0.05
    w = synth.normal_f32(11, 1, (1_000_000,), 0.02).astype(np.float64)
    assert abs(w.std() - 0.02) < 1e-4


def test_bf16_storage_matches_torch_rounding():
    f = synth.normal_f32(3, 9, (100_000,), 3.0)
    bits = synth.normal_bf16(3, 9, (100_000,), 3.0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(f).to(torch.bfloat16).float().numpy())


def test_permutation_is_a_permutation():
    p = synth.permutation(1002, synth.S_PERM, 11008)
    assert np.array_equal(np.sort(p), np.arange(11008))
    assert not np.array_equal(p, np.arange(11008))
    assert np.array_equal(p, synth.permutation(1002, synth.S_PERM, 11008))


def test_split_is_a_partition_of_the_dense_ffn():
    w = synth.make_split("t", 9, 4, 16, 48, 6, 2, act="f32", wt="f32")
    Wgate_d, Wup_d, Wdown_d = w.meta["dense"]
    perm = w.meta["perm"]
    F = w.F
    seen = np.zeros(48, dtype=int)
    for e in range(w.N):
        rows = perm[e * F:(e + 1) * F]
        seen[rows] += 1
        assert np.array_equal(w.Wgate[e], Wgate_d[rows])
        assert np.array_equal(w.Wup[e], Wup_d[rows])
        assert np.array_equal(w.Wdown[e], Wdown_d[:, rows])
    assert np.all(seen == 1)


def test_upcycled_copies_are_perturbed_base():
    w = synth.make_upcycled("t", 4, 8, 32, 16, 4, 2, perturb=1e-3, keep_base=True)
    bg = w.meta["base"][0]
    for e in range(w.N):
        d = synth.bf16_to_f32(w.Wgate[e]).astype(np.float64) - bg
        assert 2e-4 < np.abs(d).mean() < 2e-3
    assert not np.array_equal(w.Wgate[0], w.Wgate[1])
    w0 = synth.make_upcycled("t", 4, 8, 32, 16, 4, 2, perturb=0.0)
    assert all(np.array_equal(w0.Wgate[0], w0.Wgate[e]) for e in range(4))


def test_capacity_from_cf():
    assert synth.capacity_from_cf(8192, 8, 2, 4.0) == 4096
    assert synth.capacity_from_cf(8192, 8, 2, 1.0) == 1024
    assert synth.capacity_from_cf(8192, 8, 2, 1.0, count_assignments=True) == 2048
    assert synth.capacity_from_cf(10, 3, 1, 1.0) == 4


def test_skew_steers_tokens():
    w = synth.make_independent("t", 1005, 64, 256, 16, 8, 2)
    synth.apply_skew(w, n_pref=32)
    x = w.f32("x").astype(np.float64)
    logits = x @ w.Wg.astype(np.float64)
    chosen = w.meta["skew_tokens"]
    assert len(chosen) == 32
    assert np.all(np.argmax(logits[chosen], axis=1) == 0)
