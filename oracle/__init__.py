"""ORACLE -- test infrastructure only.

A plain, slow, obviously correct CPU evaluation of what the GPU path computes,
written from the pages and kept apart from the GPU path: it shares no code,
header, helper or table with ``chunkwise_gated_delta_chunk_amd`` and neither
imports the other.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import anything from here.

Contents
--------
recurrence.c / recurrence.py
    fp64 token-by-token gated delta rule over a varlen batch (GDN scalar decay,
    KDA per-key-channel decay).  The definition the chunkwise method reaches.
chunkwise_ref.py
    fp64 chunkwise Map-Reduce-Map evaluation with an explicit inverse, emitting
    per-chunk intermediates (cumulative gate, A, T = A^-1 diag(beta), M) so a
    single stage of the GPU path can be checked on its own.
meta_ref.py
    Brute-force host construction of chunk_offsets / chunk_indices from
    cu_seqlens, with the [-1, 0] sentinel.
build.py
    Compiles recurrence.c with gcc into oracle/liboracle.so.
"""
