"""The allocation-free forward (la_chunk_fwd_static, through the C ABI)
against the forward with a caller workspace (gdn_chunk_fwd / kda_chunk_fwd):
same kernels, so bit-identical outputs.  Two calls in a row on the shared
static scratch, the second with a smaller input, then a KDA call; a shape
whose workspace exceeds the array is rejected before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from synth import config, make_inputs
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def _both(inp):
    d = to_dev(inp)
    T = inp["q"].shape[0]
    H, dv = inp["H"], inp["dv"]
    N = len(inp["cu_seqlens"]) - 1
    ci, co, _ = la.build_chunk_meta(d["cu_seqlens"], T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ci, co)
    kda = inp["kda"]
    ref = la.kda_chunk_fwd if kda else la.gdn_chunk_fwd
    o1 = torch.full((T, H, dv), 3.0, device="cuda")
    h1 = torch.full((N, H, inp["dk"], dv), -2.0, device="cuda")
    o2, h2 = o1.clone(), h1.clone()
    ref(*args, h0=d["h0"], o=o1, ht=h1)
    la.chunk_fwd_static(kda, *args, h0=d["h0"], o=o2, ht=h2)
    torch.cuda.synchronize()
    return (o1, h1), (o2, h2)


def test_static_forward_matches_workspace_forward():
    big = config(1)                                   # 8 sequences, 8192 tokens, H = 16
    small = make_inputs(457, 2, 128, 128, kda=False, dtype="bf16", seed=970,
                        cu_seqlens=[0, 1, 70, 70, 200, 457], h0_std=0.1)
    kda = make_inputs(300, 3, 64, 64, kda=True, dtype="bf16", seed=971,
                      cu_seqlens=[0, 130, 300], h0_std=0.1)
    for name, inp in (("8K varlen", big), ("small", small), ("kda small", kda)):
        (o1, h1), (o2, h2) = _both(inp)
        print(f"static forward {name}: equal o {torch.equal(o1, o2)} ht {torch.equal(h1, h2)}",
              flush=True)
        assert torch.equal(o1, o2) and torch.equal(h1, h2), name


def test_static_forward_rejects_oversize():
    a = la.ChunkFwdArgs()
    a.T_max, a.N_max, a.H, a.d_k, a.d_v, a.BT, a.qkv_dtype = 65536, 1, 32, 128, 128, 64, 0
    assert la.lib().la_chunk_fwd_workspace_bytes(ctypes.byref(a), 0) > (128 << 20)
    assert la.lib().la_chunk_fwd_static(ctypes.byref(a), 0, None) == -5
    with pytest.raises(la.LinAttnError):
        T, H, d = 65536, 32, 128
        z = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
        g = torch.zeros((T, H), device="cuda")
        cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        ci, co, _ = la.build_chunk_meta(cu, T)
        la.chunk_fwd_static(False, z, z, z, g, g, cu, ci, co,
                            o=torch.empty((T, H, d), device="cuda"), output_final_state=False)
