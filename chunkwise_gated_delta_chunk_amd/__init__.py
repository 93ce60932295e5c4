"""Python binding of liblinattn.so: the MI355X varlen chunkwise gated-delta-rule
prefill forward (GDN and KDA) and its device-side chunk metadata.

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, their device pointers and the current HIP stream are handed to
the C ABI (include/linattn.h), and outputs the caller did not provide are
allocated with torch.  The library never writes rows outside every sequence
nor the final state (or dh0) of a zero-length sequence; outputs the binding
allocates start at the values those take: zero rows, ht = h0 (or 0), dh0 =
dht (or 0).  Every step of the computation runs in the library's
gfx950 kernels; if the library is missing or a call fails, an exception is
raised -- there is no other path.

Layouts (token-major varlen packing, batch 1): q, k [T_max, H, d_k];
v [T_max, H, d_v]; g [T_max, H] (GDN) or [T_max, H, d_k] (KDA); beta
[T_max, H]; cu_seqlens int32 or int64 [N_max + 1]; h0 / ht [N_max, H, d_k, d_v]
fp32; o [T_max, H, d_v] fp32 or bf16.  q, k, v are bfloat16, float16 or float32.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LinAttnError", "lib", "nt_max", "build_chunk_meta", "workspace_bytes",
    "gdn_chunk_fwd", "kda_chunk_fwd", "chunk_fwd_stages", "chunk_fwd_static", "dv_split_for",
    "seg_len_for",
    "gdn_recurrent_fwd", "kda_recurrent_fwd", "short_conv_fwd", "gdn_chunk_bwd", "kda_chunk_bwd",
    "bwd_workspace_bytes", "fork_join_events",
    "STAGE_MAP", "STAGE_REDUCE", "META_BAD_START", "META_NOT_MONOTONE",
    "META_OVER_CAPACITY", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblinattn.so")

LA_BF16, LA_F32, LA_F16 = 0, 1, 2
_DTYPES = {torch.bfloat16: LA_BF16, torch.float32: LA_F32, torch.float16: LA_F16}
_IDX = (torch.int32, torch.int64)
STAGE_MAP, STAGE_REDUCE = 1, 2
META_BAD_START, META_NOT_MONOTONE, META_OVER_CAPACITY = 1, 2, 4


class LinAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


class ChunkFwdArgs(ctypes.Structure):
    _fields_ = [
        ("T_max", ctypes.c_int32), ("N_max", ctypes.c_int32), ("H", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("BT", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32), ("dv_split", ctypes.c_int32),
        ("seg_len", ctypes.c_int32), ("H_qk", ctypes.c_int32), ("o_bf16", ctypes.c_int32),
        ("cu_seqlens_i64", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("chunk_indices", ctypes.c_void_p),
        ("chunk_offsets", ctypes.c_void_p), ("h0", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("ht", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("meta_indices", ctypes.c_void_p), ("meta_offsets", ctypes.c_void_p),
        ("meta_status", ctypes.c_void_p),
    ]


class RecurrentArgs(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int32), ("H", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32), ("H_qk", ctypes.c_int32), ("o_bf16", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("h0", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("ht", ctypes.c_void_p),
    ]


class ShortConvArgs(ctypes.Structure):
    _fields_ = [
        ("T_max", ctypes.c_int32), ("N_max", ctypes.c_int32), ("D", ctypes.c_int32),
        ("W", ctypes.c_int32), ("BT", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
        ("activation", ctypes.c_int32), ("cu_seqlens_i64", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("residual", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("chunk_indices", ctypes.c_void_p), ("h0", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("ht", ctypes.c_void_p),
    ]


class ChunkBwdArgs(ctypes.Structure):
    _fields_ = [
        ("T_max", ctypes.c_int32), ("N_max", ctypes.c_int32), ("H", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("BT", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32), ("cu_seqlens_i64", ctypes.c_int32),
        ("H_qk", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("chunk_indices", ctypes.c_void_p), ("chunk_offsets", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("dout", ctypes.c_void_p), ("dht", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("dh0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("aux_stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p),
        ("join_event", ctypes.c_void_p),
    ]


ACTIVATIONS = {None: 0, "silu": 1}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(or python chunkwise_gated_delta_chunk_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.la_nt_max.restype = ctypes.c_int64
        L.la_nt_max.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        for f in (L.build_chunk_meta, L.build_chunk_meta_i64):
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        P = ctypes.POINTER(ChunkFwdArgs)
        L.la_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.la_chunk_fwd_workspace_bytes.argtypes = [P, ctypes.c_int]
        for f in (L.gdn_chunk_fwd, L.kda_chunk_fwd):
            f.restype = ctypes.c_int
            f.argtypes = [P, ctypes.c_void_p]
        L.la_chunk_fwd_stages.restype = ctypes.c_int
        L.la_chunk_fwd_stages.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.la_chunk_fwd_static.restype = ctypes.c_int
        L.la_chunk_fwd_static.argtypes = [P, ctypes.c_int, ctypes.c_void_p]
        L.la_chunk_fwd_dv_split.restype = ctypes.c_int32
        L.la_chunk_fwd_dv_split.argtypes = [P]
        L.la_chunk_fwd_seg_len.restype = ctypes.c_int32
        L.la_chunk_fwd_seg_len.argtypes = [P]
        R = ctypes.POINTER(RecurrentArgs)
        for f in (L.gdn_recurrent_fwd, L.kda_recurrent_fwd):
            f.restype = ctypes.c_int
            f.argtypes = [R, ctypes.c_void_p]
        B = ctypes.POINTER(ChunkBwdArgs)
        L.la_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.la_chunk_bwd_workspace_bytes.argtypes = [B, ctypes.c_int]
        for f in (L.gdn_chunk_bwd, L.kda_chunk_bwd):
            f.restype = ctypes.c_int
            f.argtypes = [B, ctypes.c_void_p]
        L.la_short_conv_fwd.restype = ctypes.c_int
        L.la_short_conv_fwd.argtypes = [ctypes.POINTER(ShortConvArgs), ctypes.c_void_p]
        L.la_status_string.restype = ctypes.c_char_p
        L.la_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _status_string(s):
    try:
        return lib().la_status_string(int(s)).decode()
    except Exception:  # pragma: no cover - message only
        return "?"


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def nt_max(T_max, N_max, BT=64):
    """ceil(T_max/BT) + N_max - 1 (-1 for invalid arguments)."""
    return int(lib().la_nt_max(int(T_max), int(N_max), int(BT)))


def build_chunk_meta(cu_seqlens, T_max, BT=64, *, chunk_indices=None, chunk_offsets=None,
                     status=None, stream=None):
    """Device-side chunk metadata from cu_seqlens [N_max+1] int32 or int64.

    Returns (chunk_indices [NT_max, 2], chunk_offsets [N_max+1], status [1]),
    all int32 on cu_seqlens' device; pass preallocated tensors for capture.
    """
    _need_idx(cu_seqlens)
    N_max = cu_seqlens.numel() - 1
    NT = nt_max(T_max, N_max, BT)
    dev = cu_seqlens.device
    if chunk_indices is None:
        chunk_indices = torch.empty((max(NT, 0), 2), dtype=torch.int32, device=dev)
    if chunk_offsets is None:
        chunk_offsets = torch.empty((N_max + 1,), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=dev)
    _need(chunk_indices, "chunk_indices", torch.int32, (NT, 2), dev)
    _need(chunk_offsets, "chunk_offsets", torch.int32, (N_max + 1,), dev)
    _need(status, "status", torch.int32, (1,), dev)
    f = lib().build_chunk_meta_i64 if cu_seqlens.dtype == torch.int64 else lib().build_chunk_meta
    rc = f(_ptr(cu_seqlens), N_max, int(T_max), int(BT), _ptr(chunk_indices), _ptr(chunk_offsets),
           _ptr(status), _stream(stream))
    if rc != 0:
        raise LinAttnError(rc, "build_chunk_meta")
    return chunk_indices, chunk_offsets, status


def _need_idx(cu, dev=None):
    if cu.dtype not in _IDX:
        raise ValueError(f"cu_seqlens must be int32 or int64, got {cu.dtype}")
    _need(cu, "cu_seqlens", cu.dtype, None, dev)


def _qkv_dtype(t):
    if t.dtype not in _DTYPES:
        raise ValueError(f"q must be bfloat16, float16 or float32, got {t.dtype}")
    return _DTYPES[t.dtype]


def _shape_args(T_max, N_max, H, d_k, d_v, qkv_dtype, dv_split=0, BT=64, seg_len=0):
    a = ChunkFwdArgs()
    a.T_max, a.N_max, a.H, a.d_k, a.d_v, a.BT = T_max, N_max, H, d_k, d_v, BT
    a.qkv_dtype = _DTYPES.get(qkv_dtype, LA_F32)
    a.dv_split = dv_split
    a.seg_len = seg_len
    return a


def workspace_bytes(T_max, N_max, H, d_k, d_v, qkv_dtype, kda=False, BT=64, seg_len=0,
                    dv_split=0):
    """Forward workspace bytes (BT = 32 adds the rebuilt 64-row chunk layout;
    the images depend on the d_v split)."""
    a = _shape_args(T_max, N_max, H, d_k, d_v, qkv_dtype, dv_split, BT=BT, seg_len=seg_len)
    return int(lib().la_chunk_fwd_workspace_bytes(ctypes.byref(a), int(kda)))


def dv_split_for(T_max, N_max, H, d_k, d_v, qkv_dtype, dv_split=0, seg_len=0):
    a = _shape_args(T_max, N_max, H, d_k, d_v, qkv_dtype, dv_split, seg_len=seg_len)
    return int(lib().la_chunk_fwd_dv_split(ctypes.byref(a)))


def seg_len_for(T_max, N_max, H, d_k, d_v, qkv_dtype, seg_len=0):
    """Chunks per segment of the sequence-parallel reduce (0: one workgroup
    per sequence), after "auto"; -1 for an invalid shape."""
    a = _shape_args(T_max, N_max, H, d_k, d_v, qkv_dtype, seg_len=seg_len)
    return int(lib().la_chunk_fwd_seg_len(ctypes.byref(a)))


def _heads(q, v, what):
    """(value heads, q/k heads) of q [.., H_qk, d_k] and v [.., H, d_v]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError(f"q and v must be [{what}, heads, d]")
    H, H_qk = v.shape[1], q.shape[1]
    if H_qk < 1 or H % H_qk:
        raise ValueError(f"value heads ({H}) must be a multiple of q/k heads ({H_qk})")
    return H, H_qk


def _out(o, o_dtype, shape, dev):
    if o is None:
        # rows outside every sequence are never written by the library: an
        # output the binding allocates starts at zero there
        o = torch.zeros(shape, dtype=o_dtype or torch.float32, device=dev)
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"o must be float32 or bfloat16, got {o.dtype}")
    _need(o, "o", o.dtype, shape, dev)
    return o


def _prepare(kda, q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, h0, o, ht,
             output_final_state, workspace, scale, dv_split, seg_len, o_dtype=None, BT=64,
             static=False, build_meta=False, meta_status=None):
    _qkv_dtype(q)
    H, H_qk = _heads(q, v, "T_max")
    T_max, _, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (T_max, H_qk, d_k), dev)
    _need(v, "v", q.dtype, (T_max, H, d_v), dev)
    _need(g, "g", torch.float32, (T_max, H, d_k) if kda else (T_max, H), dev)
    _need(beta, "beta", torch.float32, (T_max, H), dev)
    _need_idx(cu_seqlens, dev)
    N_max = cu_seqlens.numel() - 1
    NT = nt_max(T_max, N_max, BT)
    _need(chunk_indices, "chunk_indices", torch.int32, (NT, 2), dev)
    _need(chunk_offsets, "chunk_offsets", torch.int32, (N_max + 1,), dev)
    if build_meta and meta_status is not None:
        _need(meta_status, "meta_status", torch.int32, (1,), dev)
    st_shape = (N_max, H, d_k, d_v)
    if h0 is not None:
        _need(h0, "h0", torch.float32, st_shape, dev)
    o = _out(o, o_dtype, (T_max, H, d_v), dev)
    if ht is None and output_final_state:
        # the library leaves ht of a zero-length sequence unwritten; a final
        # state the binding allocates holds that sequence's state, h0 (or 0)
        ht = h0.clone() if h0 is not None else torch.zeros(st_shape, dtype=torch.float32,
                                                           device=dev)
    if ht is not None:
        _need(ht, "ht", torch.float32, st_shape, dev)
    a = _shape_args(T_max, N_max, H, d_k, d_v, q.dtype, dv_split, BT=BT, seg_len=seg_len)
    a.H_qk = H_qk
    a.o_bf16 = int(o.dtype == torch.bfloat16)
    a.cu_seqlens_i64 = int(cu_seqlens.dtype == torch.int64)
    need = int(lib().la_chunk_fwd_workspace_bytes(ctypes.byref(a), int(kda)))
    if workspace is None and not static:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, dev)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (t.data_ptr() for t in (q, k, v, g, beta))
    a.cu_seqlens = cu_seqlens.data_ptr()
    a.chunk_indices = chunk_indices.data_ptr()
    a.chunk_offsets = chunk_offsets.data_ptr()
    if build_meta:
        # the call writes the layout of cu_seqlens into these two (outputs)
        a.meta_indices = chunk_indices.data_ptr()
        a.meta_offsets = chunk_offsets.data_ptr()
        a.meta_status = None if meta_status is None else meta_status.data_ptr()
    a.h0 = None if h0 is None else h0.data_ptr()
    a.o = o.data_ptr()
    a.ht = None if ht is None else ht.data_ptr()
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel()
    return a, o, ht, workspace


def _call(name, kda, stages, q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, *,
          h0=None, o=None, ht=None, output_final_state=True, workspace=None, scale=1.0,
          dv_split=0, seg_len=0, o_dtype=None, BT=64, stream=None, build_meta=False,
          meta_status=None):
    a, o, ht, workspace = _prepare(kda, q, k, v, g, beta, cu_seqlens, chunk_indices,
                                   chunk_offsets, h0, o, ht, output_final_state, workspace,
                                   scale, dv_split, seg_len, o_dtype, BT,
                                   build_meta=build_meta, meta_status=meta_status)
    L = lib()
    s = _stream(stream)
    if stages is None:
        f = L.kda_chunk_fwd if kda else L.gdn_chunk_fwd
        rc = f(ctypes.byref(a), s)
    else:
        rc = L.la_chunk_fwd_stages(ctypes.byref(a), int(kda), int(stages), s)
    if rc != 0:
        raise LinAttnError(rc, name)
    return o, ht


def gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, **kw):
    """GDN chunk forward (scalar log-decay g [T_max, H]); returns (o, ht).

    With ``build_meta=True`` (BT 64) chunk_indices and chunk_offsets are
    outputs: the call writes the layout of cu_seqlens into them (and the
    status word into ``meta_status`` if given), as build_chunk_meta would,
    inside its map kernel for up to 64 sequences."""
    return _call("gdn_chunk_fwd", False, None, q, k, v, g, beta, cu_seqlens, chunk_indices,
                 chunk_offsets, **kw)


def kda_chunk_fwd(q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, **kw):
    """KDA chunk forward (per-key-channel log-decay g [T_max, H, d_k]); returns (o, ht)."""
    return _call("kda_chunk_fwd", True, None, q, k, v, g, beta, cu_seqlens, chunk_indices,
                 chunk_offsets, **kw)


def chunk_fwd_stages(kda, stages, q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets,
                     **kw):
    """Run STAGE_MAP and/or STAGE_REDUCE of the forward (la_chunk_fwd_stages)."""
    return _call("la_chunk_fwd_stages", bool(kda), stages, q, k, v, g, beta, cu_seqlens,
                 chunk_indices, chunk_offsets, **kw)


def chunk_fwd_static(kda, q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, *,
                     h0=None, o=None, ht=None, output_final_state=True, scale=1.0, dv_split=0,
                     seg_len=0, o_dtype=None, BT=64, stream=None, build_meta=False,
                     meta_status=None):
    """The forward with the library's static device scratch as its workspace
    (la_chunk_fwd_static): for callers that cannot allocate device memory
    during the call.  Pass o (and ht) to allocate nothing here either.
    Calls that overlap on one GPU share that scratch and race."""
    a, o, ht, _ = _prepare(bool(kda), q, k, v, g, beta, cu_seqlens, chunk_indices,
                           chunk_offsets, h0, o, ht, output_final_state, None, scale, dv_split,
                           seg_len, o_dtype, BT, static=True, build_meta=build_meta,
                           meta_status=meta_status)
    rc = lib().la_chunk_fwd_static(ctypes.byref(a), int(bool(kda)), _stream(stream))
    if rc != 0:
        raise LinAttnError(rc, "la_chunk_fwd_static")
    return o, ht


def _recurrent(name, kda, q, k, v, g, beta, h0=None, o=None, ht=None, output_final_state=True,
               scale=1.0, o_dtype=None, stream=None):
    _qkv_dtype(q)
    H, H_qk = _heads(q, v, "N")
    N, _, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (N, H_qk, d_k), dev)
    _need(v, "v", q.dtype, (N, H, d_v), dev)
    _need(g, "g", torch.float32, (N, H, d_k) if kda else (N, H), dev)
    _need(beta, "beta", torch.float32, (N, H), dev)
    st_shape = (N, H, d_k, d_v)
    if h0 is not None:
        _need(h0, "h0", torch.float32, st_shape, dev)
    o = _out(o, o_dtype, (N, H, d_v), dev)
    if ht is None and output_final_state:
        ht = torch.empty(st_shape, dtype=torch.float32, device=dev)
    if ht is not None:
        _need(ht, "ht", torch.float32, st_shape, dev)
    a = RecurrentArgs()
    a.N, a.H, a.d_k, a.d_v = N, H, d_k, d_v
    a.H_qk = H_qk
    a.o_bf16 = int(o.dtype == torch.bfloat16)
    a.qkv_dtype = _qkv_dtype(q)
    a.scale = float(scale)
    a.q, a.k, a.v, a.g, a.beta = (t.data_ptr() for t in (q, k, v, g, beta))
    a.h0 = None if h0 is None else h0.data_ptr()
    a.o = o.data_ptr()
    a.ht = None if ht is None else ht.data_ptr()
    L = lib()
    f = L.kda_recurrent_fwd if kda else L.gdn_recurrent_fwd
    rc = f(ctypes.byref(a), _stream(stream))
    if rc != 0:
        raise LinAttnError(rc, name)
    return o, ht


def gdn_recurrent_fwd(q, k, v, g, beta, **kw):
    """One GDN decode step (q, k, v [N, H, d]; g, beta [N, H]); returns (o, ht).
    ht=h0 updates the state in place."""
    return _recurrent("gdn_recurrent_fwd", False, q, k, v, g, beta, **kw)


def kda_recurrent_fwd(q, k, v, g, beta, **kw):
    """One KDA decode step (g [N, H, d_k]); returns (o, ht)."""
    return _recurrent("kda_recurrent_fwd", True, q, k, v, g, beta, **kw)


def short_conv_fwd(x, weight, cu_seqlens, chunk_indices, *, bias=None, residual=None, h0=None,
                   y=None, ht=None, output_final_state=True, activation=None, BT=64,
                   stream=None):
    """Varlen causal short convolution (la_short_conv_fwd); returns (y, ht).

    x [T_max, D] bf16 / fp16 / fp32; weight [D, W] fp32; bias [D] fp32;
    residual [T_max, D] like x; h0 / ht [N_max, W-1, D] like x; activation
    None or "silu"; chunk_indices from build_chunk_meta(cu_seqlens, T_max, BT).
    """
    xdt = _qkv_dtype(x)
    if x.dim() != 2 or weight.dim() != 2:
        raise ValueError("x must be [T_max, D] and weight [D, W]")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be None or 'silu', got {activation!r}")
    T_max, D = x.shape
    W = weight.shape[1]
    dev = x.device
    _need(x, "x", x.dtype)
    _need(weight, "weight", torch.float32, (D, W), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (D,), dev)
    if residual is not None:
        _need(residual, "residual", x.dtype, (T_max, D), dev)
    _need_idx(cu_seqlens, dev)
    N_max = cu_seqlens.numel() - 1
    _need(chunk_indices, "chunk_indices", torch.int32, (nt_max(T_max, N_max, BT), 2), dev)
    st_shape = (N_max, max(W - 1, 0), D)
    if h0 is not None:
        _need(h0, "h0", x.dtype, st_shape, dev)
    if y is None:
        # rows outside every sequence are not written: zero there
        y = torch.zeros((T_max, D), dtype=x.dtype, device=dev)
    _need(y, "y", x.dtype, (T_max, D), dev)
    if ht is None and output_final_state and W > 1:
        # a zero-length sequence's history passes through unchanged
        ht = h0.clone() if h0 is not None else torch.zeros(st_shape, dtype=x.dtype, device=dev)
    if ht is not None:
        _need(ht, "ht", x.dtype, st_shape, dev)
    a = ShortConvArgs()
    a.T_max, a.N_max, a.D, a.W, a.BT = T_max, N_max, D, W, int(BT)
    a.x_dtype = xdt
    a.activation = ACTIVATIONS[activation]
    a.cu_seqlens_i64 = int(cu_seqlens.dtype == torch.int64)
    a.x, a.weight, a.y = x.data_ptr(), weight.data_ptr(), y.data_ptr()
    a.bias = None if bias is None else bias.data_ptr()
    a.residual = None if residual is None else residual.data_ptr()
    a.cu_seqlens = cu_seqlens.data_ptr()
    a.chunk_indices = chunk_indices.data_ptr()
    a.h0 = None if h0 is None else h0.data_ptr()
    a.ht = None if ht is None else ht.data_ptr()
    rc = lib().la_short_conv_fwd(ctypes.byref(a), _stream(stream))
    if rc != 0:
        raise LinAttnError(rc, "la_short_conv_fwd")
    return y, ht


def _bwd_shape(T_max, N_max, H, d_k, d_v, qkv_dtype, BT=64):
    a = ChunkBwdArgs()
    a.T_max, a.N_max, a.H, a.d_k, a.d_v, a.BT = T_max, N_max, H, d_k, d_v, BT
    a.qkv_dtype = _DTYPES.get(qkv_dtype, LA_F32)
    return a


def bwd_workspace_bytes(T_max, N_max, H, d_k, d_v, qkv_dtype, BT=64, kda=False, H_qk=0):
    a = _bwd_shape(T_max, N_max, H, d_k, d_v, qkv_dtype, BT)
    a.H_qk = H_qk
    return int(lib().la_chunk_bwd_workspace_bytes(ctypes.byref(a), int(kda)))


def gdn_chunk_bwd(*args, **kw):
    """GDN chunk backward (gdn_chunk_bwd): gradients of sum(o * dout) + sum(ht * dht).

    Arguments as gdn_chunk_fwd plus dout [T_max, H, d_v] fp32 (after
    chunk_offsets) and dht; returns (dq, dk, dv, dg, dbeta, dh0) as fp32
    tensors, dh0 None unless h0 is given or dh0 is passed.  aux_stream (a
    torch.cuda.Stream) with events = fork_join_events() runs the reverse pass
    on that stream beside the forward recompute; the caller keeps the stream
    and events to itself until the call's work is done.
    """
    return _chunk_bwd(False, *args, **kw)


def kda_chunk_bwd(*args, **kw):
    """KDA chunk backward (kda_chunk_bwd); g and dg are [T_max, H, d_k]."""
    return _chunk_bwd(True, *args, **kw)


def fork_join_events():
    """Two fresh events (fork, join) for the backward's optional second stream,
    created on the current device (a record on the current stream makes
    their handles exist)."""
    evs = (torch.cuda.Event(), torch.cuda.Event())
    for e in evs:
        e.record()
    return evs


def _handle(x, what):
    if x is None:
        return None
    if isinstance(x, torch.cuda.Stream):
        return x.cuda_stream
    if isinstance(x, torch.cuda.Event):
        h = x.cuda_event
        if not h:
            raise ValueError(f"{what} has no handle yet (record it once first)")
        return h
    return int(x)


def _chunk_bwd(kda, q, k, v, g, beta, cu_seqlens, chunk_indices, chunk_offsets, dout, *, h0=None,
               dht=None, scale=1.0, dq=None, dk=None, dv=None, dg=None, dbeta=None, dh0=None,
               workspace=None, BT=64, stream=None, aux_stream=None, events=None):
    _qkv_dtype(q)
    H, H_qk = _heads(q, v, "T_max")
    T_max, _, d_k = q.shape
    d_v = v.shape[-1]
    dev = q.device
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (T_max, H_qk, d_k), dev)
    _need(v, "v", q.dtype, (T_max, H, d_v), dev)
    g_shape = (T_max, H, d_k) if kda else (T_max, H)
    _need(g, "g", torch.float32, g_shape, dev)
    _need(beta, "beta", torch.float32, (T_max, H), dev)
    _need_idx(cu_seqlens, dev)
    N_max = cu_seqlens.numel() - 1
    NT = nt_max(T_max, N_max, BT)
    _need(chunk_indices, "chunk_indices", torch.int32, (NT, 2), dev)
    _need(chunk_offsets, "chunk_offsets", torch.int32, (N_max + 1,), dev)
    _need(dout, "dout", torch.float32, (T_max, H, d_v), dev)
    st_shape = (N_max, H, d_k, d_v)
    if h0 is not None:
        _need(h0, "h0", torch.float32, st_shape, dev)
    if dht is not None:
        _need(dht, "dht", torch.float32, st_shape, dev)

    def out(t, shape, name):
        if t is None:
            # rows outside every sequence are not written: zero gradients
            t = torch.zeros(shape, dtype=torch.float32, device=dev)
        _need(t, name, torch.float32, shape, dev)
        return t
    dq = out(dq, (T_max, H_qk, d_k), "dq")
    dk = out(dk, (T_max, H_qk, d_k), "dk")
    dv = out(dv, (T_max, H, d_v), "dv")
    dg = out(dg, g_shape, "dg")
    dbeta = out(dbeta, (T_max, H), "dbeta")
    if dh0 is None and h0 is not None:
        # dh0 of a zero-length sequence is not written; its gradient is dht
        # (the state passes through unchanged), or 0 without dht
        dh0 = dht.clone() if dht is not None else torch.zeros(st_shape, dtype=torch.float32,
                                                              device=dev)
    if dh0 is not None:
        _need(dh0, "dh0", torch.float32, st_shape, dev)
    a = _bwd_shape(T_max, N_max, H, d_k, d_v, q.dtype, BT)
    a.H_qk = H_qk
    a.cu_seqlens_i64 = int(cu_seqlens.dtype == torch.int64)
    a.scale = float(scale)
    need = int(lib().la_chunk_bwd_workspace_bytes(ctypes.byref(a), int(kda)))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    a.q, a.k, a.v, a.g, a.beta = (t.data_ptr() for t in (q, k, v, g, beta))
    a.cu_seqlens = cu_seqlens.data_ptr()
    a.chunk_indices = chunk_indices.data_ptr()
    a.chunk_offsets = chunk_offsets.data_ptr()
    a.h0 = None if h0 is None else h0.data_ptr()
    a.dout = dout.data_ptr()
    a.dht = None if dht is None else dht.data_ptr()
    a.dq, a.dk, a.dv, a.dg, a.dbeta = (t.data_ptr() for t in (dq, dk, dv, dg, dbeta))
    a.dh0 = None if dh0 is None else dh0.data_ptr()
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel()
    if (aux_stream is None) != (events is None):
        raise ValueError("aux_stream and events (fork, join) go together")
    if aux_stream is not None:
        a.aux_stream = _handle(aux_stream, "aux_stream")
        a.fork_event = _handle(events[0], "fork event")
        a.join_event = _handle(events[1], "join event")
    f = lib().kda_chunk_bwd if kda else lib().gdn_chunk_bwd
    rc = f(ctypes.byref(a), _stream(stream))
    if rc != 0:
        raise LinAttnError(rc, "kda_chunk_bwd" if kda else "gdn_chunk_bwd")
    return dq, dk, dv, dg, dbeta, dh0
