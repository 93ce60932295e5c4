"""Pins for the fp64 backward oracle (CPU only).

The oracle's gradients are checked against directional differences of the
separately pinned forward oracle (oracle/recurrence.c, fp64): for an input x,
a direction and its float32-rounded endpoints x+ and x-, the first-order
change <grad, x+ - x-> must match L(x+) - L(x-) with
L = sum(o * do) + sum(ht * dht).  The endpoints are the exact float32 values
the forward oracle reads, so input rounding cancels; the central difference
leaves a third-order truncation error.  Two closed forms complete it: with
beta = 0 the keys and values have no effect (zero gradients), and with a
single token and zero state the output is scale * beta (v q.k) k-free of g.
"""

import numpy as np
import pytest

from oracle import recurrence
from oracle.backward import gated_delta_bwd
from synth import make_inputs

CU = [0, 3, 3, 8]   # a 3-token, an empty and a 5-token sequence


def _loss(inp, do, dht, scale, **over):
    x = {key: over.get(key, inp[key]) for key in ("q", "k", "v", "g", "beta", "h0")}
    o, ht = recurrence.gated_delta_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], inp["cu_seqlens"],
                                       x["h0"], scale, kda=inp["kda"])
    rows = slice(0, inp["cu_seqlens"][-1])
    L = float(np.sum(o[rows] * do[rows]))
    ne = np.diff(inp["cu_seqlens"]) > 0
    return L + float(np.sum(ht[ne] * dht[ne]))


def _case(kda, seed):
    inp = make_inputs(CU[-1], 2, 4, 4, kda=kda, dtype="f32", seed=seed, cu_seqlens=CU, h0_std=0.5)
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(inp["v"].shape)
    dht = rng.standard_normal(inp["h0"].shape)
    return inp, do, dht


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "h0"])
def test_gradient_matches_directional_difference(kda, name):
    inp, do, dht = _case(kda, 11)
    scale = 0.7
    grads = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                            inp["h0"], do, dht, scale, kda=kda)
    rng = np.random.default_rng(99)
    x = np.asarray(inp[name], dtype=np.float64)
    d = rng.standard_normal(x.shape)
    eps = 1e-3   # truncation error ~ eps^2 relative: 1e-2 leaves ~1e-4, 1e-3 ~1e-6
    if name == "h0":
        xp, xm = x + eps * d, x - eps * d
    else:
        xp = (x + eps * d).astype(np.float32).astype(np.float64)
        xm = (x - eps * d).astype(np.float32).astype(np.float64)
    dL = _loss(inp, do, dht, scale, **{name: xp}) - _loss(inp, do, dht, scale, **{name: xm})
    g = grads["d" + name]
    lin = float(np.sum(g * (xp - xm)))
    assert abs(lin - dL) <= 1e-4 * max(abs(dL), 1e-3), (lin, dL)


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_zero_beta_keys_and_values_inert(kda):
    inp, do, dht = _case(kda, 12)
    b0 = np.zeros_like(inp["beta"])
    gr = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], b0, inp["cu_seqlens"], inp["h0"],
                         do, dht, 1.0, kda=kda)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)
    assert np.abs(gr["dbeta"]).max() > 0


def test_single_token_closed_form():
    """One token, zero state: o = scale * beta (q.k) v, so do/dv = scale beta (q.k),
    dq = scale beta (v.do) k, dk = scale beta (v.do) q, dbeta = scale (q.k)(v.do),
    dg = 0 (alpha only scales the zero state)."""
    inp = make_inputs(1, 1, 4, 3, kda=False, dtype="f32", seed=13)
    rng = np.random.default_rng(5)
    do = rng.standard_normal((1, 1, 3))
    s = 0.9
    gr = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], [0, 1], None, do,
                         None, s)
    q = np.asarray(inp["q"], dtype=np.float64)[0, 0]
    k = np.asarray(inp["k"], dtype=np.float64)[0, 0]
    v = np.asarray(inp["v"], dtype=np.float64)[0, 0]
    b = float(inp["beta"][0, 0])
    vd = float(v @ do[0, 0])
    qk = float(q @ k)
    assert np.allclose(gr["dv"][0, 0], s * b * qk * do[0, 0], rtol=1e-12, atol=1e-14)
    assert np.allclose(gr["dq"][0, 0], s * b * vd * k, rtol=1e-12, atol=1e-14)
    assert np.allclose(gr["dk"][0, 0], s * b * vd * q, rtol=1e-12, atol=1e-14)
    assert np.isclose(gr["dbeta"][0, 0], s * qk * vd, rtol=1e-12)
    assert abs(gr["dg"][0, 0]) < 1e-15
