"""Pins for the fp64 oracle (CPU only).

Each pin checks the oracle against something other than itself: a closed form
of the recurrence for a special input, an invariant, the recurrence written in
the matrix form S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T) + beta_t v_t
k_t^T, o_t = S_t q_t (the per-head recurrent state of "Empowering Hybrid
Attention Models on NPUs", section 2.1), or the independent chunkwise
evaluation.  ``test_pins_catch_planted_mistakes`` plants one mistake at a time
in a small numpy copy of the token loop and checks that some pin fails, so a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand) cannot pass them all.
"""

import numpy as np
import pytest

from oracle import chunkwise_ref, recurrence
from synth import make_inputs

TOL = 1e-11


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def oracle_fwd(q, k, v, g, beta, cu, h0=None, scale=1.0, kda=False):
    return recurrence.gated_delta_fwd(q, k, v, g, beta, cu, h0, scale, kda=kda)


# ---------------------------------------------------------------- mutants ---
def loop_fwd(q, k, v, g, beta, cu, h0=None, scale=1.0, kda=False, mut=None):
    """Plain numpy token loop used only to host planted mistakes."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [int(c) for c in cu]
    N = len(cu) - 1
    o = np.full((T, H, dv), np.nan)
    ht = np.full((N, H, dk, dv), np.nan)
    carried = np.zeros((H, dk, dv))
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        for h in range(H):
            if mut == "no_reset" and n > 0:
                S = carried[h].copy()
            else:
                S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            for t in range(bos, eos):
                tg = t - 1 if (mut == "gate_index" and t > bos) else t
                gt = g[tg, h] if not (mut == "gate_index" and t == bos) else 0.0 * g[t, h]
                a = np.exp(-gt) if mut == "exp_sign" else np.exp(gt)
                a = a * np.ones(dk) if not kda else a
                if kda and mut == "channel_flip":
                    a = a[::-1]
                kt, vt, qt, bt = k[t, h], v[t, h], q[t, h], beta[t, h]
                if mut == "decay_after":
                    u = bt * (vt - S.T @ kt)
                    S = a[:, None] * (S + np.outer(kt, u))
                else:
                    if mut == "value_axis":
                        S = S * a[None, :dv]
                    else:
                        S = a[:, None] * S
                    p = S.T @ kt
                    u = bt * (vt + p) if mut == "sign" else bt * (vt - p)
                    if mut == "no_beta_write":
                        u = vt - p
                    Sold = S
                    S = S + np.outer(kt, u)
                    if mut == "old_state_out":
                        S_read = Sold
                    else:
                        S_read = S
                if mut == "decay_after":
                    S_read = S
                o[t, h] = scale * (S_read @ qt if mut == "transposed_read" else S_read.T @ qt)
            ht[n, h] = S
            carried[h] = S
    return o, ht


MUTANTS = ["decay_after", "old_state_out", "sign", "no_beta_write", "exp_sign",
           "gate_index", "channel_flip", "value_axis", "transposed_read",
           "no_reset"]


# ------------------------------------------------------------------- pins ---
class _F32Rng:
    """numpy Generator whose draws are rounded to float32 values, the
    precision the oracle reads its inputs in."""

    def __init__(self, seed):
        self._g = np.random.default_rng(seed)

    def standard_normal(self, shape):
        return F(self._g.standard_normal(shape))

    def uniform(self, lo, hi, shape):
        return F(self._g.uniform(lo, hi, shape))

    def permutation(self, n):
        return self._g.permutation(n)

    def integers(self, lo, hi, n):
        return self._g.integers(lo, hi, n)


def F(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _rng(seed):
    return _F32Rng(seed)


def _gate(rng, shape):
    return F(-np.log1p(np.exp(-(rng.standard_normal(shape) + 1.0))))


def pin_single_token_zero_state(fwd, kda):
    """T=1 from a zero state: H = beta k v^T and o = scale beta (k.q) v."""
    rng = _rng(1)
    H, dk, dv = 2, 5, 3
    q, k = rng.standard_normal((1, H, dk)), rng.standard_normal((1, H, dk))
    v = rng.standard_normal((1, H, dv))
    g = _gate(rng, (1, H, dk) if kda else (1, H))
    b = rng.uniform(0.2, 0.9, (1, H))
    o, ht = fwd(q, k, v, g, b, [0, 1], None, 1.5, kda)
    for h in range(H):
        assert rel(ht[0, h], b[0, h] * np.outer(k[0, h], v[0, h])) < TOL
        assert rel(o[0, h], 1.5 * b[0, h] * (k[0, h] @ q[0, h]) * v[0, h]) < TOL


def pin_frozen_state(fwd, kda):
    """beta = 0 and g = 0: the state never changes, o_t = h0^T q_t (a GEMV)."""
    rng = _rng(2)
    H, dk, dv, cu = 2, 4, 4, [0, 3, 7]
    T = cu[-1]
    q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk) if kda else (T, H))
    b = np.zeros((T, H))
    h0 = rng.standard_normal((2, H, dk, dv))
    o, ht = fwd(q, k, v, g, b, cu, h0, 1.0, kda)
    assert rel(ht, h0) < TOL
    for n in range(2):
        for t in range(cu[n], cu[n + 1]):
            for h in range(H):
                assert rel(o[t, h], h0[n, h].T @ q[t, h]) < TOL


def pin_pure_decay(fwd, kda):
    """beta = 0: H_t = Diag(exp(G_t)) h0 with G_t the running sum of g."""
    rng = _rng(3)
    H, dk, dv, T = 2, 4, 4, 6
    q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = _gate(rng, (T, H, dk) if kda else (T, H))
    b = np.zeros((T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht = fwd(q, k, v, g, b, [0, T], h0, 1.0, kda)
    G = np.cumsum(g, axis=0)
    for h in range(H):
        for t in range(T):
            d = np.exp(G[t, h]) * np.ones(dk)
            assert rel(o[t, h], (d[:, None] * h0[0, h]).T @ q[t, h]) < TOL
        d = np.exp(G[T - 1, h]) * np.ones(dk)
        assert rel(ht[0, h], d[:, None] * h0[0, h]) < TOL


def pin_overwrite(fwd, kda):
    """g = 0, beta = 1, unit basis keys: each step overwrites row pi(t) with v_t."""
    rng = _rng(4)
    H, dk, dv, T = 1, 6, 4, 5
    pi = rng.permutation(dk)[:T]
    k = np.zeros((T, H, dk))
    k[np.arange(T), 0, pi] = 1.0
    sig = rng.integers(0, dk, T)
    q = np.zeros((T, H, dk))
    q[np.arange(T), 0, sig] = 1.0
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk) if kda else (T, H))
    b = np.ones((T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht = fwd(q, k, v, g, b, [0, T], h0, 1.0, kda)
    table = h0[0, 0].copy()
    for t in range(T):
        table[pi[t]] = v[t, 0]
        assert rel(o[t, 0], table[sig[t]]) < TOL
    assert rel(ht[0, 0], table) < TOL


def pin_retention(fwd, kda):
    """Zero state and keys c_t e_pi(t) on distinct channels: the delta term
    vanishes and the rule reduces to gated linear attention,
    o_t = sum_{s<=t} beta_s c_s exp(G_t - G_s)[pi(s)] q_t[pi(s)] v_s."""
    rng = _rng(5)
    H, dk, dv, T = 2, 8, 3, 7
    q = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = _gate(rng, (T, H, dk) if kda else (T, H))
    b = rng.uniform(0.1, 0.9, (T, H))
    k = np.zeros((T, H, dk))
    pis, cs = [], []
    for h in range(H):
        pi = rng.permutation(dk)[:T]
        c = rng.uniform(0.5, 2.0, T)
        k[np.arange(T), h, pi] = c
        pis.append(pi)
        cs.append(c)
    o, ht = fwd(q, k, v, g, b, [0, T], None, 1.0, kda)
    G = np.cumsum(g, axis=0)
    for h in range(H):
        pi, c = pis[h], cs[h]
        Gh = G[:, h] if kda else np.repeat(G[:, h][:, None], dk, axis=1)
        for t in range(T):
            ref = sum(b[s, h] * c[s] * np.exp(Gh[t, pi[s]] - Gh[s, pi[s]]) * q[t, h, pi[s]] * v[s, h]
                      for s in range(t + 1))
            assert rel(o[t, h], ref) < TOL
        Href = np.zeros((dk, dv))
        for s in range(T):
            Href[pi[s]] += b[s, h] * c[s] * np.exp(Gh[T - 1, pi[s]] - Gh[s, pi[s]]) * v[s, h]
        assert rel(ht[0, h], Href) < TOL


def pin_matrix_form(fwd, kda):
    """Random inputs, d_k != d_v, against the recurrence written on S (d_v x d_k):
    S <- S Diag(alpha) (I - beta k k^T) + beta v k^T, o = scale S q, ht = S^T."""
    rng = _rng(6)
    H, dk, dv, cu = 2, 5, 3, [0, 4, 9]
    T = cu[-1]
    q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk)) * 0.5
    v = rng.standard_normal((T, H, dv))
    g = _gate(rng, (T, H, dk) if kda else (T, H))
    b = rng.uniform(0.1, 0.9, (T, H))
    h0 = rng.standard_normal((2, H, dk, dv))
    o, ht = fwd(q, k, v, g, b, cu, h0, 0.7, kda)
    for n in range(2):
        for h in range(H):
            S = h0[n, h].T.copy()
            for t in range(cu[n], cu[n + 1]):
                alpha = np.exp(g[t, h]) * np.ones(dk)
                kt = k[t, h]
                S = S @ np.diag(alpha) @ (np.eye(dk) - b[t, h] * np.outer(kt, kt)) \
                    + b[t, h] * np.outer(v[t, h], kt)
                assert rel(o[t, h], 0.7 * S @ q[t, h]) < TOL
            assert rel(ht[n, h], S.T) < TOL


def pin_chunkwise(fwd, kda):
    """The chunkwise Map-Reduce-Map form (explicit inverse) agrees with the
    token recurrence for several chunk sizes, with ragged tails and varlen."""
    cu = [0, 5, 5, 23, 40]
    for BT in (4, 16, 64):
        inp = make_inputs(40, 2, 6, 5, kda=kda, dtype="f32", seed=7 + BT, cu_seqlens=cu,
                          h0_std=0.3)
        args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, inp["h0"], 1.3)
        o1, h1 = fwd(*args, kda)
        o2, h2 = chunkwise_ref.chunk_forward(*args, kda=kda, BT=BT)
        assert rel(o1, o2) < TOL
        assert np.array_equal(np.isnan(h1), np.isnan(h2))
        m = ~np.isnan(h2)
        assert rel(h1[m], h2[m]) < TOL


def pin_state_passing(fwd, kda):
    """Running [0,T) equals running [0,T1) then [T1,T) from the carried state."""
    inp = make_inputs(30, 2, 4, 6, kda=kda, dtype="f32", seed=8, h0_std=0.5)
    a = [inp[x] for x in ("q", "k", "v", "g", "beta")]
    o, ht = fwd(*a, [0, 30], inp["h0"], 1.0, kda)
    o1, h1 = fwd(*[x[:11] for x in a], [0, 11], inp["h0"], 1.0, kda)
    o2, h2 = fwd(*[x[11:] for x in a], [0, 19], h1, 1.0, kda)
    assert rel(np.concatenate([o1, o2]), o) < TOL
    assert rel(h2, ht) < TOL


def pin_varlen(fwd, kda):
    """A varlen batch equals independent per-sequence calls."""
    cu = [0, 7, 7, 12, 20]
    inp = make_inputs(20, 2, 4, 4, kda=kda, dtype="f32", seed=9, cu_seqlens=cu, h0_std=0.5)
    a = [inp[x] for x in ("q", "k", "v", "g", "beta")]
    o, ht = fwd(*a, cu, inp["h0"], 1.0, kda)
    for n in range(4):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            assert np.isnan(ht[n]).all()
            continue
        on, hn = fwd(*[x[bos:eos] for x in a], [0, eos - bos], inp["h0"][n:n + 1], 1.0, kda)
        assert rel(on, o[bos:eos]) < TOL
        assert rel(hn[0], ht[n]) < TOL


def pin_linearity(fwd, kda):
    """With beta, g fixed: (o, ht) is linear in (v, h0) jointly; o scales with scale."""
    rng = _rng(10)
    inp = make_inputs(12, 2, 4, 3, kda=kda, dtype="f32", seed=10, h0_std=0.5)
    q, k, g, b = inp["q"], inp["k"], inp["g"], inp["beta"]
    # values on a 2^-8 grid so 2*v1 - 3*v2 is exact in the float32 inputs
    v1 = np.round(inp["v"] * 256) / 256
    v2 = np.round(rng.standard_normal(inp["v"].shape) * 256) / 256
    s1, s2 = inp["h0"], rng.standard_normal(inp["h0"].shape)
    oa, ha = fwd(q, k, v1, g, b, [0, 12], s1, 1.0, kda)
    ob, hb = fwd(q, k, v2, g, b, [0, 12], s2, 1.0, kda)
    oc, hc = fwd(q, k, 2 * v1 - 3 * v2, g, b, [0, 12], 2 * s1 - 3 * s2, 1.0, kda)
    assert rel(oc, 2 * oa - 3 * ob) < 1e-10
    assert rel(hc, 2 * ha - 3 * hb) < 1e-10
    od, hd = fwd(q, k, v1, g, b, [0, 12], s1, -0.25, kda)
    assert rel(od, -0.25 * oa) < TOL
    assert rel(hd, ha) < TOL


PINS = [pin_single_token_zero_state, pin_frozen_state, pin_pure_decay, pin_overwrite,
        pin_retention, pin_matrix_form, pin_chunkwise, pin_state_passing, pin_varlen,
        pin_linearity]


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, kda):
    pin(oracle_fwd, kda)


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_unmutated_loop_passes_pins(kda):
    for pin in PINS:
        pin(lambda *a: loop_fwd(*a), kda)


@pytest.mark.parametrize("mut", MUTANTS)
def test_pins_catch_planted_mistakes(mut):
    caught = []
    for kda in (False, True):
        for pin in PINS:
            try:
                pin(lambda *a, m=mut: loop_fwd(*a, mut=m), kda)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught.append((pin.__name__, kda))
    assert caught, f"no pin detects the planted mistake {mut!r}"


def test_oracle_rejects_invalid_cu():
    inp = make_inputs(8, 1, 2, 2, kda=False, dtype="f32", seed=11)
    a = [inp[x] for x in ("q", "k", "v", "g", "beta")]
    for cu in ([1, 8], [0, 5, 3], [0, 9]):
        with pytest.raises(ValueError):
            recurrence.gated_delta_fwd(*a, cu)


def test_oracle_thread_count_invariant():
    inp = make_inputs(50, 3, 8, 8, kda=True, dtype="bf16", seed=12,
                      cu_seqlens=[0, 10, 31, 50], h0_std=0.1)
    a = [inp[x] for x in ("q", "k", "v", "g", "beta")]
    o1, h1 = recurrence.gated_delta_fwd(*a, inp["cu_seqlens"], inp["h0"], kda=True, nthreads=1)
    o4, h4 = recurrence.gated_delta_fwd(*a, inp["cu_seqlens"], inp["h0"], kda=True, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(h1, h4)
