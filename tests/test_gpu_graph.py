"""The forward captured in a HIP graph (torch.cuda.CUDAGraph drives HIP's
stream capture): moe_forward with a caller workspace, on the persistent-kernel
path and on the decode path, and moe_forward_noalloc. Every launch follows the
caller's stream and nothing allocates or synchronises, so the calls capture;
the queue counters, histograms and error word are cleared by fill kernels,
not memset nodes. Each graph is replayed several times with eager work in
between, including an eager call with other inputs on the same workspace
(or scratch array), and every replay must equal the eager result bit for
bit."""
import pytest
import torch

import synth
from gpu_util import cfg_of, log, upload, workspace
from sparse_mixture_experts_05_amd import abi

pytestmark = pytest.mark.gpu

CASES = {
    "persistent": lambda: synth.make_split("graph_fused", 71, 700, 512, 8 * 96, 8, 2, out_scale=4.0),
    "decode": lambda: synth.apply_skew(synth.make_independent("graph_dec", 72, 64, 512, 1024, 8, 2), n_pref=32),
}


def _forward(fn, cfg, d, y, ws):
    if ws is None:
        fn(cfg, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"], y)
    else:
        fn(cfg, d["x"], d["Wg"], d["Wn"], d["eps"], d["Wgate"], d["Wup"], d["Wdown"], y, ws=ws)


def _replays_match(name, noalloc):
    w = CASES[name]()
    cfg = cfg_of(w)
    d = upload(w)
    other = dict(d)
    other["x"] = d["x"].flip(0).contiguous()  # the same layer on other tokens
    fn = abi.moe_forward_noalloc if noalloc else abi.moe_forward
    ws = None if noalloc else workspace(cfg)
    y0 = torch.empty(w.T, w.H, device="cuda")
    _forward(fn, cfg, d, y0, ws)  # eager (also the first call, which sets up the scratch array)
    torch.cuda.synchronize()
    yg = torch.empty_like(y0)
    y_other = torch.empty_like(y0)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call on the capture stream
        _forward(fn, cfg, d, yg, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _forward(fn, cfg, d, yg, ws)
    for r in range(3):
        # eager work between replays: the same entry point on other inputs,
        # in the same workspace, and an unrelated product
        _forward(fn, cfg, other, y_other, ws)
        a = torch.randn(512, 512, device="cuda")
        _ = a @ a
        torch.cuda.synchronize()
        yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(yg, y0)
        log(f"[graph] {name} noalloc={noalloc} replay {r}: equal={same}")
        assert same, f"replay {r} differs from the eager result"
    assert not torch.equal(y_other, y0)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays_match_eager(name):
    _replays_match(name, noalloc=False)


def test_noalloc_forward_graph_replays_match_eager():
    _replays_match("persistent", noalloc=True)
