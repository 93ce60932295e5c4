"""Pins for the fp64 short-convolution oracle (CPU only).

Each pin checks oracle/short_conv.py against something other than itself:
numpy's own convolution on a single sequence, the impulse response, the
closed form at width 1, the carry of the final state into a continuation,
the independence of the sequences of a varlen batch, and SiLU against
scipy's logistic function.  ``test_pins_catch_planted_mistakes`` plants one
mistake at a time in a small copy of the token loop and checks that some pin
fails.
"""

import numpy as np
import pytest
from scipy.special import expit

from oracle.short_conv import short_conv_fwd
from synth import make_conv_inputs

TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# --------------------------------------------------------------- mutants ---
def loop_conv(x, w, cu, b=None, residual=None, h0=None, activation=None, mut=None):
    """Plain loop used only to host planted mistakes."""
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    W = w.shape[1]
    N = len(cu) - 1
    y = np.full((T, D), np.nan)
    ht = np.full((N, W - 1, D), np.nan)
    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        if eos == bos:
            continue
        prev = np.zeros((W - 1, D)) if h0 is None else np.array(h0[n], dtype=np.float64)
        if mut == "state_reversed":
            prev = prev[::-1]
        xs = np.concatenate([prev, x[bos:eos]])
        for t in range(eos - bos):
            z = np.zeros(D) if b is None else np.array(b, dtype=np.float64)
            if mut == "bias_after_act":
                z = np.zeros(D)
            for i in range(W):
                wi = w[:, W - 1 - i] if mut == "weights_reversed" else w[:, i]
                j = t + i + (1 if mut == "window_shift" and t + i + 1 < len(xs) else 0)
                z = z + wi * xs[j]
            if mut == "residual_before_act" and residual is not None:
                z = z + residual[bos + t]
            if activation == "silu":
                z = z / (1.0 + np.exp(-z))
            if mut == "bias_after_act" and b is not None:
                z = z + b
            if mut != "residual_before_act" and residual is not None:
                z = z + residual[bos + t]
            y[bos + t] = z
        tail = xs[len(xs) - (W - 1):]
        if mut == "state_head":
            tail = xs[:W - 1]
        ht[n] = tail
    return y, ht


MUTANTS = ["weights_reversed", "window_shift", "state_reversed", "bias_after_act",
           "residual_before_act", "state_head"]


# ------------------------------------------------------------------ pins ---
def pin_numpy_convolve(fwd):
    """One sequence, zero history, no bias, identity: per channel the full
    discrete convolution with the reversed kernel, first T terms."""
    inp = make_conv_inputs(40, 6, 4, dtype="f32", seed=1, bias=False)
    y, _ = fwd(inp["x"], inp["weight"], inp["cu_seqlens"])
    want = np.stack([np.convolve(inp["x"][:, c].astype(np.float64),
                                 inp["weight"][c, ::-1].astype(np.float64))[:40]
                     for c in range(6)], axis=1)
    return rel(y, want) <= TOL


def pin_impulse(fwd):
    """A unit impulse at t0 answers with the kernel, newest tap first."""
    W, D, T, t0 = 4, 3, 12, 5
    rng = np.random.default_rng(2)
    w = rng.standard_normal((D, W))
    x = np.zeros((T, D))
    x[t0] = 1.0
    y, _ = fwd(x, w, [0, T])
    ok = np.allclose(y[:t0], 0.0) and np.allclose(y[t0 + W:], 0.0)
    for j in range(W):
        ok = ok and np.allclose(y[t0 + j], w[:, W - 1 - j], rtol=0, atol=1e-15)
    return ok


def pin_width_one(fwd):
    """W = 1: y = act(w x + b) + r, elementwise, for every activation."""
    inp = make_conv_inputs(30, 5, 1, dtype="f32", seed=3, residual=True)
    x, w, b, r = (np.asarray(inp[k], dtype=np.float64) for k in ("x", "weight", "bias", "residual"))
    ok = True
    for act in (None, "silu"):
        y, _ = fwd(inp["x"], inp["weight"], inp["cu_seqlens"], b=inp["bias"],
                   residual=inp["residual"], activation=act)
        z = x * w[:, 0] + b
        if act == "silu":
            z = z * expit(z)
        ok = ok and rel(y, z + r) <= TOL
    return ok


def pin_state_carry(fwd):
    """Running a sequence in two parts, the first part's final state as the
    second's initial state, equals running it whole -- also when the first
    part is shorter than W - 1 -- and the final states agree."""
    inp = make_conv_inputs(50, 4, 4, dtype="f32", seed=4, residual=True, h0=True)
    kw = dict(b=inp["bias"], activation="silu")
    x, r = inp["x"], inp["residual"]
    y_all, ht_all = fwd(x, inp["weight"], [0, 50], residual=r, h0=inp["h0"], **kw)
    ok = True
    for cut in (1, 2, 17):
        y1, h1 = fwd(x[:cut], inp["weight"], [0, cut], residual=r[:cut], h0=inp["h0"], **kw)
        y2, h2 = fwd(x[cut:], inp["weight"], [0, 50 - cut], residual=r[cut:], h0=h1, **kw)
        ok = ok and rel(np.concatenate([y1, y2]), y_all) <= TOL and rel(h2, ht_all) <= TOL
    return ok


def pin_varlen_independent(fwd):
    """A varlen batch equals its sequences run one at a time."""
    cu = [0, 1, 1, 9, 30]
    inp = make_conv_inputs(34, 4, 3, dtype="f32", seed=5, cu_seqlens=cu, residual=True, h0=True)
    y, ht = fwd(inp["x"], inp["weight"], cu, b=inp["bias"], residual=inp["residual"],
                h0=inp["h0"], activation="silu")
    ok = bool(np.isnan(y[30:]).all()) and bool(np.isnan(ht[1]).all())   # tail, empty sequence
    for n in range(4):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        ys, hs = fwd(inp["x"][bos:eos], inp["weight"], [0, eos - bos], b=inp["bias"],
                     residual=inp["residual"][bos:eos], h0=inp["h0"][n:n + 1], activation="silu")
        ok = ok and rel(y[bos:eos], ys) <= TOL and rel(ht[n], hs[0]) <= TOL
    return ok


def pin_short_sequence_state(fwd):
    """A one-token sequence after history h0 = (a, b, c) leaves (b, c, x)."""
    x = np.array([[7.0]])
    h0 = np.array([[[1.0], [2.0], [3.0]]])
    _, ht = fwd(x, np.ones((1, 4)), [0, 1], h0=h0)
    return np.array_equal(ht[0, :, 0], [2.0, 3.0, 7.0])


PINS = [pin_numpy_convolve, pin_impulse, pin_width_one, pin_state_carry,
        pin_varlen_independent, pin_short_sequence_state]


def _oracle(x, w, cu, **kw):
    return short_conv_fwd(x, w, cu, **kw)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(_oracle)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_unmutated_loop_passes_pins(pin):
    assert pin(lambda *a, **k: loop_conv(*a, **k))


@pytest.mark.parametrize("mut", MUTANTS)
def test_pins_catch_planted_mistakes(mut):
    fails = [p.__name__ for p in PINS if not p(lambda *a, **k: loop_conv(*a, mut=mut, **k))]
    assert fails, f"no pin catches {mut}"


def test_silu_matches_logistic():
    z = np.linspace(-30, 30, 601)
    from oracle.short_conv import silu
    assert rel(silu(z), z * expit(z)) <= 1e-15
