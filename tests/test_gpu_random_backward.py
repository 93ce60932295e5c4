"""GPU: the chunk backward on seeded random varlen layouts, against the
reverse-mode fp64 oracle.

Each case draws GDN or KDA; bf16, fp16 or fp32 inputs (d = 64 or 128; fp32
at 64); 1 to 3 heads; 1 to 6 sequences mixing empty, one-token, exact
multiples of the 64-row chunk and arbitrary lengths below 200; with or
without h0 and dht; scale 1, 0.5 or d^-1/2.  Every gradient must meet the
dtype's tolerance relative to its own largest reference value.  Where a
reference gradient is exactly zero (dg of a lone token with no initial
state: the gate then reaches nothing), the scale it is measured against is
floored at 1e-4 of the case's largest reference gradient, so rounding that
cancels to ~1e-9 of that is not read as a relative error.
"""

import numpy as np
import pytest

from oracle.backward import gated_delta_bwd
from synth import make_inputs
from tests.helpers import TOL
from tests.test_gpu_backward import run_bwd

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(80_000 + i)
    kda = bool(rng.integers(2))
    dt = ["bf16", "f16", "f32"][rng.integers(3)]
    d = 64 if dt == "f32" else int(rng.choice([64, 128]))
    H = int(rng.integers(1, 4))
    N = int(rng.integers(1, 7))
    lens = rng.integers(0, 200, N)
    lens[rng.random(N) < 0.2] = 0
    lens[rng.random(N) < 0.15] = 1
    lens[rng.random(N) < 0.15] = 64 * int(rng.integers(1, 3))
    if lens.sum() == 0:
        lens[0] = 7
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    inp = make_inputs(int(cu[-1]), H, d, d, kda=kda, dtype=dt, seed=int(rng.integers(1 << 30)),
                      cu_seqlens=cu, h0_std=0.1)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32) if rng.random() < 0.5 else None
    with_h0 = bool(rng.random() < 0.7)
    scale = float(rng.choice([1.0, 0.5, d ** -0.5]))
    return inp, cu, do, dht, with_h0, scale


@pytest.mark.parametrize("i", range(40))
def test_random_backward(i):
    inp, cu, do, dht, with_h0, scale = _case(i)
    print(f"random backward {i}: kda={inp['kda']} {inp['dtype']} d={inp['dk']} H={inp['H']} "
          f"N={len(cu) - 1} T={int(cu[-1])} dht={dht is not None} h0={with_h0}", flush=True)
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu,
                          inp["h0"] if with_h0 else None, do, dht, scale, kda=inp["kda"])
    got = run_bwd(inp, do, dht, scale, with_h0=with_h0)
    rows = slice(0, int(cu[-1]))
    ne = np.diff(cu) > 0
    pairs = {key: (got[key].cpu().numpy()[rows], ref[key][rows])
             for key in ("dq", "dk", "dv", "dg", "dbeta")}
    if got["dh0"] is not None:
        pairs["dh0"] = (got["dh0"].cpu().numpy()[ne], ref["dh0"][ne])
    top = max(float(np.abs(r).max()) if r.size else 0.0 for _, r in pairs.values())
    errs = {}
    for key, (x, r) in pairs.items():
        if r.size == 0:
            continue
        den = max(float(np.abs(r).max()), 1e-4 * top, 1e-30)
        errs[key] = float(np.abs(x.astype(np.float64) - r).max() / den)
    print("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    tol = TOL[inp["dtype"]]
    assert all(np.isfinite(v) and v <= tol for v in errs.values()), errs
