"""Seeded synthetic inputs for the varlen gated-delta-rule chunk forward.

This module is shared by the CPU oracle side (tests) and the GPU side (tests,
bench).  It holds only the input recipe: random draws, L2 normalisation of q/k,
the log-sigmoid gate and sigmoid beta, rounding to bf16, and the sequence-length
layouts.  None of the method's arithmetic (decay, delta update, chunking) lives
here.

The workload shapes follow the pages: a 64-token chunk (BT=64) and the varlen
packing of the FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA
Prefill and Training Paths on Ascend NPUs", section "Fixed-capacity execution");
T=2048/H=10/C=64 and 65,536 tokens from "Empowering Hybrid Attention Models on
NPUs" (section 2.3, Figure 4; section 7.5).  No public dataset is involved.

All arrays are numpy; floating arrays are float32 holding values that are exact
in the storage dtype ("bf16" values are bf16-representable), so both sides read
identical numbers.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "make_inputs", "config", "bucket_layout", "bucket_replay_layout",
    "CONFIG_NAMES",
]


def bf16_round(x):
    """Round float32 values to the nearest bf16 value (ties to even); float32 out.

    On the bit pattern u: add 0x7FFF plus the lowest kept bit, clear the low 16
    bits.  For every non-NaN u the sum stays below 2^32, so uint32 arithmetic
    is exact; NaNs are restored afterwards (the sum can carry out of a NaN's
    payload)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r &= np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def _l2norm(x):
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / np.maximum(n, 1e-6)


def _store(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)   # nearest fp16
    return bf16_round(x) if dtype == "bf16" else x


def make_inputs(T, H, dk, dv, *, kda, dtype, seed, cu_seqlens=None, h0_std=None,
                round_gate=False, n_seqs=None, cuts=None, rng=None):
    """Draw one batch of inputs in a fixed order: q, k, v, g, beta, (cuts), h0.

    q, k ~ N(0,1) then L2-normalised per (token, head); v ~ N(0,1);
    beta = sigmoid(N(0,1)); g = logsigmoid(N(0,1) + 3), per (token, head) for
    GDN and per (token, head, key channel) for KDA.  q/k/v are rounded to the
    storage dtype ("bf16", "f16" or "f32"); g and beta stay float32 unless
    ``round_gate`` asks for bf16-valued gates.

    ``cuts`` is an optional callable ``rng -> cu_seqlens`` drawn after beta, so a
    layout can come from the same stream; otherwise ``cu_seqlens`` (or one
    sequence of length T) is used.  h0 ~ N(0, h0_std) of shape [N, H, dk, dv]
    when ``h0_std`` is given, else None.  ``rng`` continues a given generator
    instead of seeding a new one.
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_l2norm(rng.standard_normal((T, H, dk))), dtype)
    k = _store(_l2norm(rng.standard_normal((T, H, dk))), dtype)
    v = _store(rng.standard_normal((T, H, dv)), dtype)
    gshape = (T, H, dk) if kda else (T, H)
    x = rng.standard_normal(gshape) + 3.0
    g = (-np.logaddexp(0.0, -x)).astype(np.float32)          # logsigmoid(x)
    b = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    if round_gate:
        g = bf16_round(g)
        b = bf16_round(b)
    if cuts is not None:
        cu = np.asarray(cuts(rng), dtype=np.int32)
    elif cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int32)
    else:
        cu = np.array([0, T], dtype=np.int32)
    N = len(cu) - 1
    h0 = None
    if h0_std is not None:
        h0 = (rng.standard_normal((N, H, dk, dv)) * h0_std).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=b, cu_seqlens=cu, h0=h0,
                T=T, H=H, dk=dk, dv=dv, kda=bool(kda), dtype=dtype)


def make_conv_inputs(T, D, W, *, dtype, seed, cu_seqlens=None, bias=True, residual=False,
                     h0=False):
    """Inputs of the short convolution, drawn in a fixed order: x, weight,
    bias, residual, h0.

    x ~ N(0,1) [T, D] rounded to the storage dtype; weight ~ N(0, 0.5)
    [D, W] float32; bias ~ N(0, 0.1) [D] float32; residual ~ N(0,1) [T, D] and
    h0 ~ N(0,1) [N, W-1, D], both in the storage dtype (h0 holds past inputs).
    ``cu_seqlens`` defaults to one sequence of length T.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _store(rng.standard_normal((T, D)), dtype)
    w = (rng.standard_normal((D, W)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(D) * 0.1).astype(np.float32) if bias else None
    r = _store(rng.standard_normal((T, D)), dtype) if residual else None
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    s0 = _store(rng.standard_normal((N, W - 1, D)), dtype) if h0 else None
    return dict(x=x, weight=w, bias=b, residual=r, h0=s0, cu_seqlens=cu, T=T, D=D, W=W,
                dtype=dtype)


def _uniform_cuts(T, n):
    """n sequences covering [0, T): n-1 distinct cut points uniform on {1..T-1}."""
    def draw(rng):
        pts = np.sort(rng.choice(np.arange(1, T), size=n - 1, replace=False))
        return np.concatenate([[0], pts, [T]]).astype(np.int32)
    return draw


def bucket_layout(rng, T_max, N_max, n=None):
    """A fixed-capacity bucket layout: cu_seqlens of shape [N_max+1].

    N ~ U{1..N_max} (unless ``n`` is given); proportions ~ Dirichlet(1_N);
    len_i = max(1, floor(p_i * T_max)); any excess over T_max is taken from the
    longest sequence; slots N+1..N_max repeat the total (zero-length tails).
    """
    if n is None:
        n = int(rng.integers(1, N_max + 1))
    p = rng.dirichlet(np.ones(n))
    lens = np.maximum(1, np.floor(p * T_max).astype(np.int64))
    excess = int(lens.sum()) - T_max
    if excess > 0:
        lens[int(np.argmax(lens))] -= excess
    cu = np.zeros(N_max + 1, dtype=np.int64)
    cu[1:n + 1] = np.cumsum(lens)
    cu[n + 1:] = cu[n]
    return cu.astype(np.int32)


BUCKET_T_MAX, BUCKET_N_MAX = 16384, 64


def bucket_replay_layout(replay):
    """The layout of bucket replay ``replay`` (workload 3) alone: the first
    draw of that replay's stream, so it needs none of the inputs drawn after
    it."""
    rng = np.random.Generator(np.random.PCG64(3000 + replay))
    return bucket_layout(rng, BUCKET_T_MAX, BUCKET_N_MAX)


CONFIG_NAMES = {
    0: "gdn fp32 T=256 N=1 H=2 d=64",
    1: "gdn bf16 varlen T=8192 N=8 H=16 d=128 (h0~N(0,0.1))",
    2: "kda bf16 T=4096 N=1 H=16 d=128",
    3: "gdn bf16 bucket T_max=16384 N_max=64 H=32 d=128",
    4: "gdn/kda bf16 T=65536 (or 2048) N=1 H=10 d=128",
}


def config(idx, *, replay=0, kda=None, T=None):
    """Inputs of one of the five workloads, seeded by the workload index.

    0: GDN fp32, one sequence T=256, H=2, d=64, zero state, seed 0.
    1: GDN bf16 q/k/v, fp32 g/beta/state, H=16, d=128, T=8192 cut into 8
       sequences by 7 uniform cut points, h0 ~ N(0, 0.1), seed 1.
    2: KDA bf16 (q/k/v and bf16-valued g/beta), one sequence T=4096, H=16,
       d=128, zero state, seed 2.
    3: fixed-capacity bucket T_max=16384, N_max=64, GDN bf16, H=32, d=128,
       no initial state; replay r draws a fresh layout (bucket_replay_layout)
       and then its inputs from one stream seeded 3000+r (padding rows hold
       ordinary non-zero data).
    4: GDN (kda=False) or KDA (kda=True) bf16, one sequence, H=10, d=128,
       T=65536 (default) or T=2048, zero state, seed 4.
    """
    if idx == 0:
        return make_inputs(256, 2, 64, 64, kda=False, dtype="f32", seed=0)
    if idx == 1:
        return make_inputs(8192, 16, 128, 128, kda=False, dtype="bf16", seed=1,
                           cuts=_uniform_cuts(8192, 8), h0_std=0.1)
    if idx == 2:
        return make_inputs(4096, 16, 128, 128, kda=True, dtype="bf16", seed=2,
                           round_gate=True)
    if idx == 3:
        rng = np.random.Generator(np.random.PCG64(3000 + replay))
        cu = bucket_layout(rng, BUCKET_T_MAX, BUCKET_N_MAX)
        return make_inputs(BUCKET_T_MAX, 32, 128, 128, kda=False, dtype="bf16",
                           seed=3000 + replay, cu_seqlens=cu, rng=rng)
    if idx == 4:
        T = 65536 if T is None else T
        return make_inputs(T, 10, 128, 128, kda=bool(kda), dtype="bf16", seed=4)
    raise ValueError(f"no workload {idx}")
