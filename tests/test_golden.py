"""Hand-derived cases (tests/golden/hand_cases.json): each output has a closed
form derived from the cited equation; the oracle must reproduce it."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "hand_cases.json")))["cases"]

_NS = {"exp": math.exp, "log": math.log, "sqrt": math.sqrt,
       "f32": lambda v: float(np.float32(v)), "__builtins__": {}}


def _ev(e):
    return float(eval(e, _NS)) if isinstance(e, str) else float(e)


def _workload(c):
    T, H, F, N, k = c["T"], c["H"], c["F"], c["N"], c["k"]
    a = lambda v, shape: np.ascontiguousarray(np.array(v, np.float32).reshape(shape))
    z = lambda shape: np.zeros(shape, np.float32)
    return synth.Workload(c["name"], T, H, F, N, k, c["capacity"], c["order"], c["noisy"], False,
                          c["out_scale"], "f32", "f32", a(c["x"], (T, H)), a(c["Wg"], (H, N)),
                          a(c["Wn"], (H, N)) if "Wn" in c else None,
                          a(c["eps"], (T, N)) if "eps" in c else None,
                          a(c["Wgate"], (N, F, H)) if "Wgate" in c else z((N, F, H)),
                          a(c["Wup"], (N, F, H)) if "Wup" in c else z((N, F, H)),
                          a(c["Wdown"], (N, H, F)) if "Wdown" in c else z((N, H, F)))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case(case):
    w = _workload(case)
    out = oracle.forward(w, h_round=oracle.H_EXACT)
    ex = case["expect"]
    for key in ("topk_idx", "counts", "kept", "offsets", "slot", "row_token"):
        if key in ex:
            assert np.array_equal(np.asarray(out[key]).reshape(-1), np.asarray(ex[key]).reshape(-1)), key
    for key, okey in (("topk_w", "topk_w"), ("y", "y64"), ("H", "H"), ("logits", "logits"),
                      ("min_gap", "min_gap")):
        if key in ex:
            want = np.vectorize(_ev, otypes=[float])(np.array(ex[key], dtype=object))
            got = np.asarray(out[okey], np.float64).reshape(want.shape)
            np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15, err_msg=key)
