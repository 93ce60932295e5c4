"""ORACLE (test infrastructure only): fp64 varlen causal short convolution.

The FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA Prefill
and Training Paths on Ascend NPUs", sections "Proposed API" and "Step 3: GDN
and short-convolution graph support") names the short convolution of the
layer path (projection, short convolution, then the chunk attention) and the
cases it must cover -- dense and varlen inputs, bias, activation and residual,
initial and final states, fixed chunk metadata -- without printing its
formula.  The reading taken here is the usual depthwise causal one: for
channel c of a sequence with tokens x_0 .. x_{L-1} and kernel width W,

    y_t[c] = act( b[c] + sum_{i=0}^{W-1} w[c, i] * x_{t-(W-1)+i}[c] ) + r_t[c]

where x_p for p < 0 is row W-1+p of the sequence's initial state (the last
W-1 inputs before it; zero when there is none), act is the identity or SiLU
(z * sigmoid(z)), and r the optional residual.  The final state is the W-1
inputs ending at the sequence's last token, reaching back into the initial
state when the sequence is shorter than W-1.  Sequences never see each
other's tokens.

Shapes: x, r, y [T, D]; w [D, W]; b [D]; states [N, W-1, D].
"""

import numpy as np


def silu(z):
    return z / (1.0 + np.exp(-z))


def short_conv_fwd(x, w, cu_seqlens, b=None, residual=None, h0=None, activation=None):
    """Return (y [T, D] fp64, ht [N, W-1, D] fp64).

    Rows of y outside every sequence stay NaN, and so does ht of an empty
    sequence (neither is defined by the operation).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, D = x.shape
    W = w.shape[1]
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    y = np.full((T, D), np.nan)
    ht = np.full((N, W - 1, D), np.nan)
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        # the sequence's inputs preceded by its initial state
        prev = np.zeros((W - 1, D)) if h0 is None else np.asarray(h0[n], dtype=np.float64)
        xs = np.concatenate([prev, x[bos:eos]], axis=0)     # xs[W-1+t] = x_t
        for t in range(eos - bos):
            z = np.zeros(D) if b is None else np.asarray(b, dtype=np.float64).copy()
            for i in range(W):
                z = z + w[:, i] * xs[t + i]
            if activation == "silu":
                z = silu(z)
            if residual is not None:
                z = z + np.asarray(residual[bos + t], dtype=np.float64)
            y[bos + t] = z
        ht[n] = xs[len(xs) - (W - 1):]
    return y, ht
