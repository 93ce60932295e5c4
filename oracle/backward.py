"""ORACLE (test infrastructure only): fp64 gradients of the gated delta rule.

The forward is the token recurrence of "Empowering Hybrid Attention Models on
NPUs" (section 2.1), in the step order oracle/recurrence.c documents (H = S^T):
    H <- Diag(alpha_t) H;  u = beta_t (v_t - H^T k_t);  H <- H + k_t u^T;
    o_t = scale H^T q_t,   alpha_t = exp(g_t)
over the sequences of cu_seqlens, each from its own initial state.  The FLA
graph-capture RFC puts the backward of the chunk path in scope (sections
"Scope" and "Step 3"), with gradients for q, k, v, the gate, beta and the
initial state.  Here they are the gradients of
    L = sum(o * do) + sum(ht * dht)
obtained by reverse-mode differentiation (torch.autograd, float64, CPU) of
the token loop written out below; no chunking, no reordering.
"""

import numpy as np
import torch


def gated_delta_bwd(q, k, v, g, beta, cu_seqlens, h0, do, dht=None, scale=1.0, kda=False):
    """Return dict of fp64 numpy gradients: dq, dk, dv, dg, dbeta, dh0.

    Shapes as the forward: q, k [T, H, dk]; v, do [T, H, dv]; g [T, H] (GDN)
    or [T, H, dk] (KDA); beta [T, H]; h0, dht [N, H, dk, dv] or None.  Rows
    outside every sequence get zero gradients; dh0 of an empty sequence is
    zero (its final state is not an output).
    """
    f64 = torch.float64
    t = {name: torch.tensor(np.asarray(x, dtype=np.float64), dtype=f64, requires_grad=True)
         for name, x in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta))}
    T, H, dk = t["q"].shape
    dv = t["v"].shape[2]
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    h0_t = (torch.zeros((N, H, dk, dv), dtype=f64) if h0 is None
            else torch.tensor(np.asarray(h0, dtype=np.float64), dtype=f64))
    h0_t.requires_grad_(True)
    do_t = torch.tensor(np.asarray(do, dtype=np.float64), dtype=f64)
    dht_t = None if dht is None else torch.tensor(np.asarray(dht, dtype=np.float64), dtype=f64)
    loss = torch.zeros((), dtype=f64)
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        S = h0_t[n]                                   # [H, dk, dv]
        for s in range(bos, eos):
            a = torch.exp(t["g"][s])                  # [H] or [H, dk]
            S = S * (a[:, :, None] if kda else a[:, None, None])
            kt, vt, qt, bt = t["k"][s], t["v"][s], t["q"][s], t["beta"][s]
            p = torch.einsum("hkv,hk->hv", S, kt)
            u = bt[:, None] * (vt - p)
            S = S + kt[:, :, None] * u[:, None, :]
            o = scale * torch.einsum("hkv,hk->hv", S, qt)
            loss = loss + (o * do_t[s]).sum()
        if dht_t is not None:
            loss = loss + (S * dht_t[n]).sum()
    loss.backward()
    out = {f"d{name}": (x.grad.numpy().copy() if x.grad is not None else np.zeros(x.shape))
           for name, x in t.items()}
    out["dh0"] = h0_t.grad.numpy().copy()
    out["dbeta"] = out.pop("dbeta")
    return out
