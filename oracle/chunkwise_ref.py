"""ORACLE (test infrastructure only): fp64 chunkwise Map-Reduce-Map evaluation.

The chunkwise form of the gated delta rule, evaluated literally with numpy in
fp64, chunk after chunk, with an explicit matrix inverse.  It is a second,
independent algorithm for the same result as recurrence.c, and it exposes the
per-chunk intermediates that the GPU path's chunk-parallel stage produces.

Method ("Empowering Hybrid Attention Models on NPUs", section 2.1: Map
precomputes chunk-local transforms, Reduce carries the state across chunks,
the final Map forms token outputs; section 5 names the shared-input GEMMs
K S, Q S, K K^T, Q K^T and factors A^-1 out of W = A^-1 K).  The FLA RFC
("[RFC] Add Graph Capture Support for FLA Prefill and Training Paths on Ascend
NPUs", "Step 3") lists the stages as gate/chunk cumsum -> forward intra ->
recompute_w_u -> forward h -> forward o.

For one chunk of C rows with entering state H0 = S^T ([dk, dv]) and gate rows
g_r (vector over dk; GDN broadcasts its scalar), derived from the token
recurrence by unrolling C steps:
    G_r   = sum_{s<=r} g_s                      (gate / chunk cumsum)
    A     = I + strict_lower(beta_r * sum_i k_ri k_si exp(G_ri - G_si))
    M     = lower_incl(sum_i q_ri k_si exp(G_ri - G_si))
    T     = A^-1 diag(beta)                     (forward intra)
    U     = T (V - (K * exp(G)) H0)             (state-corrected values)
    O     = scale * ((Q * exp(G)) H0 + M U)     (forward o)
    H_C   = diag(exp(G_C)) H0 + (K * exp(G_C - G))^T U   (forward h)
"""

import numpy as np


def _chunk(K, Q, V, gl, B, S, scale, kda):
    C, dk = K.shape
    G = np.cumsum(gl, axis=0)
    Gm = G if kda else np.repeat(G[:, None], dk, axis=1)
    E = np.exp(Gm[:, None, :] - Gm[None, :, :])            # [r, s, i]
    KK = np.einsum("ri,si,rsi->rs", K, K, E)
    QK = np.einsum("ri,si,rsi->rs", Q, K, E)
    A = np.eye(C) + np.tril(B[:, None] * KK, -1)
    M = np.tril(QK)
    T = np.linalg.inv(A) @ np.diag(B)
    Kd = K * np.exp(Gm)
    Qd = Q * np.exp(Gm)
    Kb = K * np.exp(Gm[-1][None, :] - Gm)
    U = T @ (V - Kd @ S)
    O = scale * (Qd @ S + M @ U)
    Sn = np.exp(Gm[-1])[:, None] * S + Kb.T @ U
    return O, Sn, dict(G=G, A=A, T=T, M=M, U=U, H0=S.copy())


def chunk_forward(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, *,
                  kda=False, BT=64, keep=False):
    """fp64 chunkwise forward over a varlen batch.

    Same arguments and results as recurrence.gated_delta_fwd.  With keep=True
    also returns a dict mapping (slot, head) -> per-chunk intermediates, where
    slot enumerates chunks sequence-major then chunk-minor (the chunk_indices
    order).
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    o = np.full((T, H, dv), np.nan)
    ht = np.full((N, H, dk, dv), np.nan)
    inter = {}
    slot = 0
    for n in range(N):
        bos, eos = cu[n], cu[n + 1]
        if eos == bos:
            continue
        S = (np.zeros((H, dk, dv)) if h0 is None
             else np.asarray(h0[n], dtype=np.float64).copy())
        for c0 in range(bos, eos, BT):
            rows = slice(c0, min(c0 + BT, eos))
            for h in range(H):
                O, S[h], it = _chunk(k[rows, h], q[rows, h], v[rows, h],
                                     g[rows, h], beta[rows, h], S[h], scale, kda)
                o[rows, h] = O
                if keep:
                    inter[(slot, h)] = it
            slot += 1
        ht[n] = S
    return (o, ht, inter) if keep else (o, ht)
