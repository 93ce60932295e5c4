"""C-ABI checks that need no GPU: the library loads, exports every function
include/linattn.h declares, and rejects bad arguments on the host before
anything is enqueued (every case below fails a host check, so no launch is
attempted)."""

import ctypes
import os
import re

import pytest

import chunkwise_gated_delta_chunk_amd as la
from oracle import meta_ref

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "linattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(",
                                 text, flags=re.M)) - {"defined"})


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"build_chunk_meta", "build_chunk_meta_i64", "gdn_chunk_fwd", "kda_chunk_fwd", "la_nt_max",
            "la_chunk_fwd_workspace_bytes", "la_status_string"} <= set(names)
    L = ctypes.CDLL(la.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("T,N,BT", [(16384, 64, 64), (8192, 8, 64), (1, 1, 64), (65, 3, 32),
                                    (0, 3, 64), (5, 0, 64)])
def test_nt_max_matches_formula(T, N, BT):
    want = meta_ref.nt_max(T, N, BT) if T >= 1 and N >= 1 else -1
    assert la.nt_max(T, N, BT) == want


def test_status_strings():
    for s in range(0, -8, -1):
        assert la.lib().la_status_string(s)
    assert la.lib().la_status_string(99) == b"unknown status"


def _args(**kw):
    a = la.ChunkFwdArgs()
    a.T_max, a.N_max, a.H, a.d_k, a.d_v, a.BT, a.qkv_dtype = 256, 2, 2, 64, 64, 64, 0
    a.scale = 1.0
    fake = 0x100000  # 256-aligned, never dereferenced: every case fails before launch
    for f in ("q", "k", "v", "g", "beta", "cu_seqlens", "chunk_indices", "chunk_offsets", "o",
              "workspace"):
        setattr(a, f, fake)
    a.workspace_bytes = 1 << 30
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BAD = [
    ("null q", dict(q=None), -1),
    ("null o", dict(o=None), -1),
    ("null metadata", dict(chunk_offsets=None), -1),
    ("T_max 0", dict(T_max=0), -2),
    ("N_max 0", dict(N_max=0), -2),
    ("H 0", dict(H=0), -2),
    ("dtype 7", dict(qkv_dtype=7), -3),
    ("BT 16", dict(BT=16), -4),
    ("d 96", dict(d_k=96, d_v=96), -4),
    ("d_k != d_v", dict(d_v=128), -4),
    ("fp32 d 128", dict(qkv_dtype=1, d_k=128, d_v=128), -4),
    ("dv_split 3", dict(dv_split=3), -4),
    ("dv_split 8", dict(dv_split=8), -4),
    ("dv_split too fine", dict(dv_split=4), -4),
    ("no workspace", dict(workspace=None), -5),
    ("workspace small", dict(workspace_bytes=100), -5),
    ("workspace misaligned", dict(workspace=0x100010), -5),
    ("q misaligned", dict(q=0x100008), -2),
    ("ht partly over h0", dict(h0=0x200000, ht=0x200000 + 4096), -6),
    ("o misaligned", dict(o=0x100008), -2),
    ("H_qk not dividing H", dict(H=6, H_qk=4), -2),
    ("H_qk negative", dict(H_qk=-1), -2),
    ("o_bf16 2", dict(o_bf16=2), -3),
    ("cu_seqlens_i64 2", dict(cu_seqlens_i64=2), -3),
    ("fp16 d 96", dict(qkv_dtype=2, d_k=96, d_v=96), -4),
    ("fp16 BT 48", dict(qkv_dtype=2, BT=48), -4),
    ("fp32 segmented", dict(qkv_dtype=1, seg_len=4), -4),
    ("own layout without offsets", dict(meta_indices=0x300000), -1),
    ("own layout at BT 32", dict(meta_indices=0x300000, meta_offsets=0x300100, BT=32), -4),
    ("own layout, still no workspace", dict(meta_indices=0x300000, meta_offsets=0x300100,
                                            chunk_indices=None, chunk_offsets=None,
                                            workspace=None), -5),
]


@pytest.mark.parametrize("name,kw,code", BAD, ids=[b[0] for b in BAD])
def test_forward_rejects_on_host(name, kw, code):
    a = _args(**kw)
    L = la.lib()
    assert L.gdn_chunk_fwd(ctypes.byref(a), None) == code
    assert L.kda_chunk_fwd(ctypes.byref(a), None) == code
    assert L.la_chunk_fwd_stages(ctypes.byref(a), 0, 3, None) == code


def test_forward_null_args_and_bad_stages():
    L = la.lib()
    assert L.gdn_chunk_fwd(None, None) == -1
    a = _args(workspace_bytes=100)
    assert L.la_chunk_fwd_stages(ctypes.byref(a), 0, 0, None) == -4
    assert L.la_chunk_fwd_stages(ctypes.byref(a), 0, 4, None) == -4


@pytest.mark.parametrize("fn", ["build_chunk_meta", "build_chunk_meta_i64"])
def test_meta_rejects_on_host(fn):
    f = getattr(la.lib(), fn)
    p = ctypes.c_void_p(0x100000)
    assert f(None, 2, 256, 64, p, p, None, None) == -1
    assert f(p, 2, 256, 64, None, p, None, None) == -1
    assert f(p, 0, 256, 64, p, p, None, None) == -2
    assert f(p, 8193, 256, 64, p, p, None, None) == -2
    assert f(p, 2, 0, 64, p, p, None, None) == -2
    for bt in (16, 48, 128, 0):  # 32 and 64 are built
        assert f(p, 2, 256, bt, p, p, None, None) == -4


def test_workspace_size_and_split():
    import torch
    for (T, N, H, d, dt, esz, raw) in [(8192, 8, 16, 128, torch.bfloat16, 2, True),
                                       (256, 1, 2, 64, torch.float32, 4, False),
                                       (16384, 64, 32, 128, torch.bfloat16, 2, True)]:
        cells = meta_ref.nt_max(T, N, 64) * H
        # one image per cell: K, Q, [K^T: KDA or fp32], Tn, M, vec padded to
        # 1 KiB; GDN with 16-bit inputs in 32- or 64-column slices (raw)
        # stores no K and Q (its reduce stages them itself)
        vec = -(-(192 + d) * 4 // 1024) * 1024
        kt = 64 * d * esz
        gdn = (0 if raw else 2 * 64 * d * esz) + (kt if esz == 4 else 0) + \
            2 * 64 * 64 * esz + vec
        assert la.workspace_bytes(T, N, H, d, d, dt) == cells * gdn
        kda = 2 * 64 * d * esz + kt + 2 * 64 * 64 * esz + vec
        assert la.workspace_bytes(T, N, H, d, d, dt, kda=True) == cells * kda
    # a 64-column split of the first shape stages K and Q from the raw rows
    # too; a 128-column one stores them again
    cells = meta_ref.nt_max(8192, 8, 64) * 16
    raw = (2 * 64 * 64 * 2 + 2048) * cells
    full = (2 * 64 * 128 * 2 + 2 * 64 * 64 * 2 + 2048) * cells
    assert la.workspace_bytes(8192, 8, 16, 128, 128, torch.bfloat16, dv_split=2) == raw
    assert la.workspace_bytes(8192, 8, 16, 128, 128, torch.bfloat16, dv_split=1) == full
    assert la.workspace_bytes(0, 1, 1, 64, 64, torch.bfloat16) == 0
    # 64 columns per workgroup, 32 when that leaves at most one workgroup per
    # CU (256 of them)
    assert la.dv_split_for(8192, 8, 16, 128, 128, torch.bfloat16) == 4
    assert la.dv_split_for(8192, 8, 17, 128, 128, torch.bfloat16) == 2
    assert la.dv_split_for(16384, 64, 32, 128, 128, torch.bfloat16) == 2
    assert la.dv_split_for(65536, 1, 10, 128, 128, torch.bfloat16, seg_len=-1) == 4
    # segmented: 64-column slices (13 x 10 x 8 = 1040 workgroups at 32)
    assert la.dv_split_for(65536, 1, 10, 128, 128, torch.bfloat16) == 2
    assert la.dv_split_for(4096, 1, 2, 64, 64, torch.bfloat16) == 2
    assert la.dv_split_for(256, 1, 2, 64, 64, torch.float32) == 2
    assert la.dv_split_for(4096, 512, 2, 64, 64, torch.float32) == 1
    assert la.dv_split_for(256, 1, 2, 64, 64, torch.float32, dv_split=1) == 1


def test_segment_length_choice():
    """Sequence-parallel reduce: auto segments only bf16 buckets whose
    (sequence, head) units cannot fill half the CUs at 64 columns, about
    NT_max * H * (d_v / 64) / 256 chunks per segment (at least 4), when a
    T_max-token sequence would have 3 or more segments."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    assert la.seg_len_for(65536, 1, 10, 128, 128, bf) == 80      # 1024 * 10 * 2 / 256
    assert la.seg_len_for(4096, 1, 16, 128, 128, bf) == 8        # 64 * 16 * 2 / 256
    assert la.seg_len_for(2048, 1, 10, 128, 128, bf) == 8        # 2.5 -> at least 8
    assert la.seg_len_for(1024, 1, 10, 128, 128, bf) == 0        # 16 chunks < 3 x 8
    assert la.seg_len_for(8192, 8, 16, 128, 128, bf) == 0        # 256 units: plain
    assert la.seg_len_for(16384, 64, 32, 128, 128, bf) == 0
    assert la.seg_len_for(512, 1, 2, 128, 128, bf) == 0          # 8 chunks < 3 segments
    # segmented slices: 32 columns while the first pass has <= 512 workgroups
    assert la.dv_split_for(2048, 1, 10, 128, 128, bf) == 4       # 4 x 10 x 8 = 320
    assert la.dv_split_for(4096, 1, 16, 128, 128, bf) == 2       # 8 x 16 x 8 = 1024
    assert la.seg_len_for(65536, 1, 10, 64, 64, f32) == 0        # fp32: plain
    assert la.seg_len_for(65536, 1, 10, 128, 128, bf, seg_len=-1) == 0
    assert la.seg_len_for(4096, 3, 2, 128, 128, bf, seg_len=5) == 5
    assert la.seg_len_for(4096, 3, 2, 64, 64, f32, seg_len=5) == -1      # unsupported
    assert la.seg_len_for(4096, 65, 2, 128, 128, bf, seg_len=5) == -1    # N_max > 64
    assert la.seg_len_for(4096, 3, 2, 128, 128, bf, seg_len=-2) == -1


def test_workspace_with_segments():
    """Segmented: the images, then hin, dlt and the transition images, each
    [segment slots][H][d_k][d_v] x 4 bytes, segment slots =
    ceil(T_max / (64 L)) + N_max - 1."""
    import torch
    T, N, H, d, L = 4096, 3, 2, 128, 5
    plain = la.workspace_bytes(T, N, H, d, d, torch.bfloat16, seg_len=-1)
    seg = la.workspace_bytes(T, N, H, d, d, torch.bfloat16, seg_len=L)
    ns = -(-T // (64 * L)) + N - 1
    assert seg - plain == 3 * ns * H * d * d * 4
    # auto: 12 units at 64 columns, NT_max = 66 -> 8 chunks per segment
    assert la.seg_len_for(T, N, H, d, d, torch.bfloat16) == 8
    assert la.workspace_bytes(T, N, H, d, d, torch.bfloat16) == \
        la.workspace_bytes(T, N, H, d, d, torch.bfloat16, seg_len=8)


def _rargs(**kw):
    a = la.RecurrentArgs()
    a.N, a.H, a.d_k, a.d_v, a.qkv_dtype, a.scale = 4, 2, 128, 128, 0, 1.0
    fake = 0x100000  # never dereferenced: every case fails before launch
    for f in ("q", "k", "v", "g", "beta", "o"):
        setattr(a, f, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


RBAD = [
    ("null q", dict(q=None), -1),
    ("null beta", dict(beta=None), -1),
    ("null o", dict(o=None), -1),
    ("N 0", dict(N=0), -2),
    ("H 0", dict(H=0), -2),
    ("N*H too big", dict(N=1 << 20, H=1 << 12), -2),
    ("dtype 5", dict(qkv_dtype=5), -3),
    ("fp16 d 96", dict(qkv_dtype=2, d_k=96, d_v=96), -4),
    ("d 96", dict(d_k=96, d_v=96), -4),
    ("d_k != d_v", dict(d_v=64), -4),
    ("v misaligned", dict(v=0x100004), -2),
    ("h0 misaligned", dict(h0=0x100008), -2),
    ("ht partly over h0", dict(h0=0x200000, ht=0x200000 + 4096), -6),
    ("H_qk not dividing H", dict(H=6, H_qk=4), -2),
    ("o_bf16 2", dict(o_bf16=2), -3),
]


@pytest.mark.parametrize("name,kw,code", RBAD, ids=[b[0] for b in RBAD])
def test_recurrent_rejects_on_host(name, kw, code):
    a = _rargs(**kw)
    L = la.lib()
    assert L.gdn_recurrent_fwd(ctypes.byref(a), None) == code
    assert L.kda_recurrent_fwd(ctypes.byref(a), None) == code
    assert L.gdn_recurrent_fwd(None, None) == -1


def _cargs(**kw):
    a = la.ShortConvArgs()
    a.T_max, a.N_max, a.D, a.W, a.BT, a.x_dtype = 256, 2, 64, 4, 64, 0
    fake = 0x100000  # never dereferenced: every case fails before launch
    for f in ("x", "weight", "cu_seqlens", "chunk_indices"):
        setattr(a, f, fake)
    a.y = 0x8000000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


CBAD = [
    ("null x", dict(x=None), -1),
    ("null weight", dict(weight=None), -1),
    ("null y", dict(y=None), -1),
    ("null chunk_indices", dict(chunk_indices=None), -1),
    ("dtype 3", dict(x_dtype=3), -3),
    ("activation 2", dict(activation=2), -3),
    ("cu_seqlens_i64 2", dict(cu_seqlens_i64=2), -3),
    ("W 0", dict(W=0), -4),
    ("W 5", dict(W=5), -4),
    ("BT 16", dict(BT=16), -4),
    ("T_max 0", dict(T_max=0), -2),
    ("D 0", dict(D=0), -2),
    ("D 12 bf16", dict(D=12), -2),
    ("D 6 fp32", dict(D=6, x_dtype=1), -2),
    ("x misaligned", dict(x=0x100008), -2),
    ("bias misaligned", dict(bias=0x100004), -2),
    ("y over x", dict(y=0x100000 + 64), -6),
    ("y partly over residual", dict(residual=0x9000000, y=0x9000000 + 32), -6),
    ("ht partly over h0", dict(h0=0x200000, ht=0x200000 + 128), -6),
]


@pytest.mark.parametrize("name,kw,code", CBAD, ids=[b[0] for b in CBAD])
def test_short_conv_rejects_on_host(name, kw, code):
    a = _cargs(**kw)
    assert la.lib().la_short_conv_fwd(ctypes.byref(a), None) == code
    assert la.lib().la_short_conv_fwd(None, None) == -1


def _bargs(**kw):
    a = la.ChunkBwdArgs()
    a.T_max, a.N_max, a.H, a.d_k, a.d_v, a.BT, a.qkv_dtype = 256, 2, 2, 64, 64, 64, 0
    a.scale = 1.0
    fake = 0x100000  # never dereferenced: every case fails before launch
    for f in ("q", "k", "v", "g", "beta", "cu_seqlens", "chunk_indices", "chunk_offsets", "dout",
              "dq", "dk", "dv", "dg", "dbeta", "workspace"):
        setattr(a, f, fake)
    a.workspace_bytes = 1 << 34
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BBAD = [
    ("null dout", dict(dout=None), -1),
    ("null dq", dict(dq=None), -1),
    ("null dbeta", dict(dbeta=None), -1),
    ("dtype 4", dict(qkv_dtype=4), -3),
    ("BT 16", dict(BT=16), -4),
    ("d 96", dict(d_k=96, d_v=96), -4),
    ("no workspace", dict(workspace=None), -5),
    ("workspace small", dict(workspace_bytes=1000), -5),
    ("q misaligned", dict(q=0x100008), -2),
    ("dout misaligned", dict(dout=0x100004), -2),
    ("dq misaligned", dict(dq=0x100008), -2),
    ("dk misaligned", dict(dk=0x100004), -2),
    ("dv misaligned", dict(dv=0x100008), -2),
    ("H 0", dict(H=0), -2),
    ("aux stream without events", dict(aux_stream=0x100000), -1),
    ("events without aux stream", dict(fork_event=0x100000, join_event=0x100000), -1),
]


@pytest.mark.parametrize("name,kw,code", BBAD, ids=[b[0] for b in BBAD])
def test_backward_rejects_on_host(name, kw, code):
    a = _bargs(**kw)
    L = la.lib()
    assert L.gdn_chunk_bwd(ctypes.byref(a), None) == code
    assert L.kda_chunk_bwd(ctypes.byref(a), None) == code
    assert L.gdn_chunk_bwd(None, None) == -1


def test_backward_workspace_size():
    """[forward images][entering states][leaving gradients][prep][partials],
    each region rounded up to 256 bytes."""
    import torch
    T, N, H, d = 1000, 3, 2, 128
    cells = meta_ref.nt_max(T, N, 64) * H
    up = lambda x: -(-x // 256) * 256
    for kda in (False, True):
        # the recompute reduces 16-bit inputs in 32-column slices
        img = la.workspace_bytes(T, N, H, d, d, torch.bfloat16, kda=kda, seg_len=-1,
                                 dv_split=d // 32)
        prep = (12544 + 8192 if not kda else 12352 + 64 * d + 8192) * 4   # + bf16 halves of M, A~
        part = (192 * d + 8192 + 256) * 4
        want = up(img) + 2 * up(cells * d * d * 4) + up(cells * prep) + up(cells * part)
        assert la.bwd_workspace_bytes(T, N, H, d, d, torch.bfloat16, kda=kda) == want


def test_workspace_with_bt32_layout():
    """BT = 32: the forward's workspace also holds the rebuilt 64-row layout
    (chunk_indices [NT_max(64)][2], chunk_offsets [N_max+1], a status word)."""
    import torch
    T, N, H, d = 4096, 3, 2, 128
    base = la.workspace_bytes(T, N, H, d, d, torch.bfloat16, seg_len=-1)
    b32 = la.workspace_bytes(T, N, H, d, d, torch.bfloat16, BT=32, seg_len=-1)
    assert b32 - base == (2 * meta_ref.nt_max(T, N, 64) + N + 2) * 4
