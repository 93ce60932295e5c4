"""ORACLE (test infrastructure only): brute-force chunk metadata on the host.

Follows the FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA
Prefill and Training Paths on Ascend NPUs"), section "Fixed-capacity
execution": a bucket (T_max, N_max, BT) has at most
NT_max = ceil(T_max / BT) + N_max - 1 chunks; cu_seqlens has shape [N_max+1],
chunk_indices [NT_max, 2] holds (sequence, chunk-within-sequence) pairs and
unused slots hold the sentinel [-1, 0]; chunk_offsets [N_max+1] holds the
first slot of each sequence.  Section "Device-side metadata" says the same
layout is regenerated from cu_seqlens on every replay.

Readings where the page is silent: slots are enumerated sequence-major, then
chunk-minor (slot chunk_offsets[n] + i_t holds (n, i_t)); zero-length
sequences own no slot; an invalid cu_seqlens (cu[0] != 0, a decrease, or a
total above T_max) yields a non-zero status bit set, all-sentinel
chunk_indices and all-zero chunk_offsets.
"""

import numpy as np

STATUS_BAD_START = 1      # cu_seqlens[0] != 0
STATUS_NOT_MONOTONE = 2   # cu_seqlens[n+1] < cu_seqlens[n] for some n
STATUS_OVER_CAPACITY = 4  # cu_seqlens[N_max] > T_max


def nt_max(T_max, N_max, BT):
    """Chunk capacity of a bucket: ceil(T_max/BT) + N_max - 1."""
    return -(-int(T_max) // int(BT)) + int(N_max) - 1


def status_of(cu, N_max, T_max):
    cu = [int(x) for x in cu]
    s = 0
    if cu[0] != 0:
        s |= STATUS_BAD_START
    for n in range(N_max):
        if cu[n + 1] < cu[n]:
            s |= STATUS_NOT_MONOTONE
    if cu[N_max] > T_max:
        s |= STATUS_OVER_CAPACITY
    return s


def chunk_meta(cu, N_max, T_max, BT):
    """Return (chunk_indices [NT_max,2] int32, chunk_offsets [N_max+1] int32, status)."""
    cu = [int(x) for x in cu]
    assert len(cu) == N_max + 1
    NT = nt_max(T_max, N_max, BT)
    idx = np.empty((NT, 2), dtype=np.int32)
    idx[:, 0] = -1
    idx[:, 1] = 0
    off = np.zeros(N_max + 1, dtype=np.int32)
    st = status_of(cu, N_max, T_max)
    if st:
        return idx, off, st
    slot = 0
    for n in range(N_max):
        length = cu[n + 1] - cu[n]
        nchunks = 0
        while nchunks * BT < length:     # ceil(length / BT), by counting
            idx[slot, 0] = n
            idx[slot, 1] = nchunks
            slot += 1
            nchunks += 1
        off[n + 1] = off[n] + nchunks
    assert slot <= NT
    return idx, off, st
