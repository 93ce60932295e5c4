"""GPU: the forward building its own chunk layout (``build_meta=True``, the
ABI's meta_indices / meta_offsets / meta_status).

The layout the call writes must equal build_chunk_meta's and the oracle's
(meta_ref) bit for bit, for valid and invalid cu_seqlens, up to 64 sequences
(derived in the map kernel's prologue) and beyond (the metadata kernel runs
first).  o and ht must equal those of the same call on build_chunk_meta's
layout bit for bit (the same kernels on the same cells), and the oracle to
the usual tolerance on the larger cases.
"""

import json
import os

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from oracle import meta_ref
from synth import bucket_layout, config, make_inputs
from tests.helpers import TOL, compare, run_oracle, to_dev

pytestmark = pytest.mark.gpu

CANARY = -7


def _say(*a):
    print(*a, flush=True)


def _fwd(inp):
    return la.kda_chunk_fwd if inp["kda"] else la.gdn_chunk_fwd


def _both(inp, cu_dev=None, cu_dtype=torch.int32, **kw):
    """(o, ht) on build_chunk_meta's layout, then (o, ht, ci, co, st) of the
    call that builds its own layout into canary-filled arrays."""
    d = to_dev(inp, cu_dtype=cu_dtype)
    cu = d["cu_seqlens"] if cu_dev is None else cu_dev
    T = inp["q"].shape[0]
    N = cu.numel() - 1
    ci0, co0, _ = la.build_chunk_meta(cu, T)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], cu)
    o_nan = lambda: torch.full((T, inp["H"], inp["dv"]), float("nan"), device="cuda")  # noqa: E731
    o0, ht0 = _fwd(inp)(*args, ci0, co0, h0=d["h0"], o=o_nan(), **kw)
    NT = la.nt_max(T, N)
    ci = torch.full((NT, 2), CANARY, dtype=torch.int32, device="cuda")
    co = torch.full((N + 1,), CANARY, dtype=torch.int32, device="cuda")
    st = torch.full((1,), CANARY, dtype=torch.int32, device="cuda")
    o1, ht1 = _fwd(inp)(*args, ci, co, h0=d["h0"], o=o_nan(), build_meta=True, meta_status=st,
                        **kw)
    torch.cuda.synchronize()
    return (o0, ht0), (o1, ht1, ci, co, st)


def _check_layout(cu, T_max, ci, co, st):
    N = len(cu) - 1
    ref_i, ref_o, ref_s = meta_ref.chunk_meta([int(x) for x in cu], N, T_max, 64)
    assert np.array_equal(ci.cpu().numpy(), ref_i), "chunk_indices"
    assert np.array_equal(co.cpu().numpy(), ref_o), "chunk_offsets"
    assert int(st.item()) == ref_s, "status"
    return ref_s


def _same(a, b):
    return torch.equal(torch.nan_to_num(a, nan=1e30), torch.nan_to_num(b, nan=1e30))


@pytest.mark.parametrize("kind", ["gdn_bf16", "kda_bf16", "gdn_f32", "kda_f32"])
@pytest.mark.parametrize("N", [1, 7, 64, 65, 100])
def test_fused_layout_random(kind, N):
    kda = kind.startswith("kda")
    dt = kind.split("_")[1]
    d = 64 if dt == "f32" else 128
    rng = np.random.default_rng(500 + N + 7 * kda + 13 * (dt == "f32"))
    T = 1500
    cu = bucket_layout(rng, T, N)
    inp = make_inputs(T, 2, d, d, kda=kda, dtype=dt, seed=N, cu_seqlens=cu, h0_std=0.1)
    _say("fused layout", kind, "N", N, "chunks", int(((np.diff(cu) + 63) // 64).sum()))
    (o0, ht0), (o1, ht1, ci, co, st) = _both(inp)
    assert _check_layout(cu, T, ci, co, st) == 0
    assert _same(o0, o1) and torch.equal(ht0, ht1)


def test_fused_layout_golden_cases():
    """The metadata golden cases at BT = 64, valid and invalid: the written
    layout matches, and an invalid layout writes no output row."""
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "meta_cases.json")))
    for c in cases["cases"]:
        if c["BT"] != 64:
            continue
        for idx in (torch.int32, torch.int64):
            T = c["T_max"]
            _say("fused golden", c["name"], idx)
            inp = make_inputs(T, 2, 64, 64, kda=False, dtype="bf16", seed=3, h0_std=None)
            cu_dev = torch.tensor(c["cu"], dtype=idx, device="cuda")
            (o0, ht0), (o1, ht1, ci, co, st) = _both(inp, cu_dev=cu_dev, cu_dtype=idx)
            s = _check_layout(c["cu"], T, ci, co, st)
            assert _same(o0, o1)
            if s != 0:
                assert torch.isnan(o1).all(), "an invalid layout writes no output row"


def test_fused_layout_int64_and_stages():
    """int64 cu_seqlens, and the map and reduce as separate stage calls (the
    reduce reads the offsets its map call wrote)."""
    rng = np.random.default_rng(77)
    T = 2000
    cu = bucket_layout(rng, T, 12)
    inp = make_inputs(T, 2, 128, 128, kda=False, dtype="bf16", seed=9, cu_seqlens=cu,
                      h0_std=0.1)
    (o0, ht0), (o1, ht1, ci, co, st) = _both(inp, cu_dtype=torch.int64)
    _check_layout(cu, T, ci, co, st)
    assert _same(o0, o1) and torch.equal(ht0, ht1)
    d = to_dev(inp)
    N = len(cu) - 1
    ci2 = torch.full((la.nt_max(T, N), 2), CANARY, dtype=torch.int32, device="cuda")
    co2 = torch.full((N + 1,), CANARY, dtype=torch.int32, device="cuda")
    ws = torch.empty((la.workspace_bytes(T, N, 2, 128, 128, torch.bfloat16),), dtype=torch.uint8,
                     device="cuda")
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ci2, co2)
    o2 = torch.full_like(o0, float("nan"))
    ht2 = d["h0"].clone()  # zero-length sequences keep h0, as the binding's own ht does
    kw = dict(h0=d["h0"], o=o2, ht=ht2, workspace=ws, build_meta=True)
    la.chunk_fwd_stages(False, la.STAGE_MAP, *args, **kw)
    la.chunk_fwd_stages(False, la.STAGE_REDUCE, *args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ci2, ci) and torch.equal(co2, co)
    assert _same(o2, o0) and torch.equal(ht2, ht0)


@pytest.mark.parametrize("cfg", [1, 2])
def test_fused_layout_workloads(cfg):
    """The 8K varlen GDN and 4K KDA workloads: bitwise equal to the call on
    build_chunk_meta's layout and at parity with the oracle (2 heads)."""
    inp = config(cfg)
    _say("fused workload", cfg)
    (o0, ht0), (o1, ht1, ci, co, st) = _both(inp)
    _check_layout(inp["cu_seqlens"], inp["q"].shape[0], ci, co, st)
    assert _same(o0, o1) and torch.equal(ht0, ht1)
    heads = [0, inp["H"] - 1]
    o_ref, ht_ref = run_oracle(inp, heads=heads)
    eo, eh, tol = compare(inp, o1, ht1, o_ref, ht_ref, heads=heads)
    _say(f"config{cfg} fused o {eo:.2e} ht {eh:.2e}")
    assert eo <= TOL[inp["dtype"]] and eh <= TOL[inp["dtype"]]


def test_fused_layout_graph_replays():
    """One captured call that builds its layout, replayed on fresh layouts
    copied into the static cu_seqlens: every replay equals an eager call on
    build_chunk_meta's layout."""
    T_max, N_max, H, d = 4096, 16, 4, 128
    bf = torch.bfloat16
    inp = make_inputs(T_max, H, d, d, kda=False, dtype="bf16", seed=21, h0_std=None)
    dv = to_dev(inp)
    cu = torch.zeros((N_max + 1,), dtype=torch.int32, device="cuda")
    NT = la.nt_max(T_max, N_max)
    ci = torch.zeros((NT, 2), dtype=torch.int32, device="cuda")
    co = torch.zeros((N_max + 1,), dtype=torch.int32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    o = torch.zeros((T_max, H, d), device="cuda")
    ht = torch.zeros((N_max, H, d, d), device="cuda")
    ws = torch.empty((la.workspace_bytes(T_max, N_max, H, d, d, bf),), dtype=torch.uint8,
                     device="cuda")
    args = (dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], cu, ci, co)
    kw = dict(o=o, ht=ht, workspace=ws, build_meta=True, meta_status=st)
    rng = np.random.default_rng(31)
    cu.copy_(torch.from_numpy(bucket_layout(rng, T_max, N_max)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.gdn_chunk_fwd(*args, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.gdn_chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    for r in range(4):
        lay = bucket_layout(rng, T_max, N_max)
        cu.copy_(torch.from_numpy(lay))
        o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        o_g, ht_g = o.clone(), ht.clone()
        ci0, co0, _ = la.build_chunk_meta(cu, T_max)
        o_e, ht_e = la.gdn_chunk_fwd(*args[:6], ci0, co0, o=torch.full_like(o, float("nan")),
                                     ht=ht.clone(), workspace=ws)
        torch.cuda.synchronize()
        _say("fused replay", r, "sequences", int((np.diff(lay) > 0).sum()))
        _check_layout(lay, T_max, ci, co, st)
        n = int(lay[-1])
        assert torch.equal(o_g[:n], o_e[:n])
        ne = np.diff(lay) > 0
        assert torch.equal(ht_g[torch.from_numpy(ne).cuda()], ht_e[torch.from_numpy(ne).cuda()])
