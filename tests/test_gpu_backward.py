"""GPU parity of the GDN and KDA chunk backward against the fp64 oracle
(oracle/backward.py: reverse-mode gradients of the token recurrence).

Bar, per gradient (dq, dk, dv, dg, dbeta over the rows of real tokens; dh0
over non-empty sequences): max |x - ref| / max |ref| <= 2e-3 for 16-bit
inputs and 1e-4 for fp32 inputs.  Rows outside every sequence are never
written.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from oracle.backward import gated_delta_bwd
from synth import make_inputs
from tests.helpers import TOL, TORCH_DT, rel_err

pytestmark = pytest.mark.gpu

SMALL_CU = [0, 1, 64, 64, 200, 333, 460]   # one token, exact chunk, empty, tails


def _say(*a):
    print(*a, flush=True)


def run_bwd(inp, do, dht, scale, *, with_h0=True, idx=torch.int32, fill=None):
    tdt = TORCH_DT[inp["dtype"]]
    d = {x: torch.from_numpy(inp[x]).cuda().to(tdt).contiguous() for x in ("q", "k", "v")}
    g = torch.from_numpy(inp["g"]).cuda().contiguous()
    b = torch.from_numpy(inp["beta"]).cuda().contiguous()
    cu = torch.from_numpy(np.asarray(inp["cu_seqlens"], dtype=np.int64)).cuda().to(idx)
    T = inp["q"].shape[0]
    ci, co, _ = la.build_chunk_meta(cu, T)
    h0 = torch.from_numpy(inp["h0"]).cuda() if (with_h0 and inp["h0"] is not None) else None
    dout = torch.from_numpy(np.asarray(do, dtype=np.float32)).cuda()
    dh = None if dht is None else torch.from_numpy(np.asarray(dht, dtype=np.float32)).cuda()
    outs = {}
    if fill is not None:
        H, dk, dv = inp["H"], inp["dk"], inp["dv"]
        outs = dict(dq=torch.full((T, H, dk), fill, device="cuda"),
                    dk=torch.full((T, H, dk), fill, device="cuda"),
                    dv=torch.full((T, H, dv), fill, device="cuda"),
                    dg=torch.full(inp["g"].shape, fill, device="cuda"),
                    dbeta=torch.full((T, H), fill, device="cuda"))
    f = la.kda_chunk_bwd if inp["kda"] else la.gdn_chunk_bwd
    res = f(d["q"], d["k"], d["v"], g, b, cu, ci, co, dout, h0=h0, dht=dh, scale=scale, **outs)
    torch.cuda.synchronize()
    return dict(zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), res))


def compare(inp, got, ref):
    cu = np.asarray(inp["cu_seqlens"])
    rows = slice(0, int(cu[-1]))
    ne = np.diff(cu) > 0
    errs = {}
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        errs[key] = rel_err(got[key].cpu().numpy()[rows], ref[key][rows])
    if got["dh0"] is not None:
        errs["dh0"] = rel_err(got["dh0"].cpu().numpy()[ne], ref["dh0"][ne])
    return errs


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 64)])
def test_backward_matches_oracle(kda, dtype, d):
    inp = make_inputs(SMALL_CU[-1], 3, d, d, kda=kda, dtype=dtype, seed=700 + d,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    rng = np.random.default_rng(701)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], SMALL_CU,
                          inp["h0"], do, dht, 0.75, kda=kda)
    got = run_bwd(inp, do, dht, 0.75)
    errs = compare(inp, got, ref)
    _say(f"bwd {'kda' if kda else 'gdn'} {dtype} d={d}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    tol = TOL[dtype]
    assert all(v <= tol for v in errs.values()), errs


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_backward_no_state_no_dht_and_padding_untouched(kda):
    T_max = 300
    cu = [0, 70, 70, 250]
    inp = make_inputs(T_max, 2, 64, 64, kda=kda, dtype="bf16", seed=710, cu_seqlens=cu)
    rng = np.random.default_rng(711)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, None, do, None,
                          kda=kda)
    got = run_bwd(inp, do, None, 1.0, fill=7.0)
    errs = compare(inp, got, ref)
    _say("bwd no state: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert bool((got[key][250:] == 7.0).all()), key


def test_backward_int64_offsets_and_determinism():
    inp = make_inputs(SMALL_CU[-1], 2, 128, 128, kda=False, dtype="bf16", seed=720,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    rng = np.random.default_rng(721)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    a = run_bwd(inp, do, dht, 1.0)
    b = run_bwd(inp, do, dht, 1.0, idx=torch.int64)
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[key][:460], b[key][:460]), key
    assert torch.equal(a["dh0"][ne], b["dh0"][ne])


def test_backward_config1_sampled_heads():
    """The 8K varlen workload's layout and inputs (H = 16, d = 128, bf16), the
    oracle on one head (its autograd tape holds every token's state)."""
    from synth import config
    inp = config(1)
    rng = np.random.default_rng(730)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    got = run_bwd(inp, do, None, 1.0)
    heads = [11]
    sub = {x: np.ascontiguousarray(inp[x][:, heads]) for x in ("q", "k", "v", "g", "beta")}
    ref = gated_delta_bwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], inp["cu_seqlens"],
                          inp["h0"][:, heads], do[:, heads], None, 1.0)
    errs = {}
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        errs[key] = rel_err(got[key].cpu().numpy()[:, heads], ref[key])
    errs["dh0"] = rel_err(got["dh0"].cpu().numpy()[:, heads], ref["dh0"])
    _say("bwd config1 head 11: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_backward_kda_config2_sampled_head():
    """The KDA workload's inputs (one sequence T = 4096, H = 16, d = 128, bf16,
    bf16-valued gates), the oracle on one head."""
    from synth import config
    inp = config(2)
    rng = np.random.default_rng(740)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    got = run_bwd(inp, do, None, 1.0)
    heads = [5]
    sub = {x: np.ascontiguousarray(inp[x][:, heads]) for x in ("q", "k", "v", "g", "beta")}
    ref = gated_delta_bwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], inp["cu_seqlens"],
                          None, do[:, heads], None, 1.0, kda=True)
    errs = {key: rel_err(got[key].cpu().numpy()[:, heads], ref[key])
            for key in ("dq", "dk", "dv", "dg", "dbeta")}
    _say("bwd kda config2 head 5: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("H_qk", [1, 2])
def test_backward_grouped_value_heads(kda, H_qk):
    """q, k with H_qk heads shared by H = 4 value heads: dq, dk of a q/k head
    are the sums of the oracle's gradients over its group (the oracle runs on
    q, k repeated per value head)."""
    from tests.helpers import gva
    inp = make_inputs(SMALL_CU[-1], 4, 64, 64, kda=kda, dtype="bf16", seed=760 + H_qk,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    small, full = gva(inp, H_qk)
    rng = np.random.default_rng(761)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    ref = gated_delta_bwd(full["q"], full["k"], full["v"], full["g"], full["beta"], SMALL_CU,
                          full["h0"], do, dht, 1.0, kda=kda)
    G = 4 // H_qk
    T = SMALL_CU[-1]
    for key in ("dq", "dk"):
        ref[key] = ref[key].reshape(T, H_qk, G, 64).sum(axis=2)
    got = run_bwd(small, do, dht, 1.0)
    errs = compare(small, got, ref)
    _say(f"bwd gva kda={kda} H_qk={H_qk}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("dscale", [1e-6, 1e5])
def test_backward_gradient_scale(kda, dscale):
    """The bf16 path splits every non-key operand into bf16 high and low
    halves, which keep fp32's exponent range: a loss scaled by 1e-6 (a mean
    over many tokens) or 1e5 (loss scaling) must keep the same relative
    accuracy.  The oracle's gradients are linear in (dout, dht)."""
    inp = make_inputs(SMALL_CU[-1], 2, 128, 128, kda=kda, dtype="bf16", seed=770,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    rng = np.random.default_rng(771)
    do = rng.standard_normal(inp["v"].shape) * dscale
    dht = rng.standard_normal(inp["h0"].shape) * dscale
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], SMALL_CU,
                          inp["h0"], do, dht, 1.0, kda=kda)
    got = run_bwd(inp, do.astype(np.float32), dht.astype(np.float32), 1.0)
    errs = compare(inp, got, ref)
    _say(f"bwd scale {dscale:g} kda={kda}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_backward_kda_strong_decay():
    """KDA gates of -2 .. -6 per token and channel: the cumulative gate falls
    by up to ~380 over a chunk, so exp(-G) overflows fp32.  The block
    factorisation keeps every exponential factor at most one; the gradients
    must stay finite and match the oracle."""
    inp = make_inputs(SMALL_CU[-1], 2, 64, 64, kda=True, dtype="bf16", seed=780,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    rng = np.random.default_rng(781)
    inp["g"] = (-rng.uniform(2.0, 6.0, size=inp["g"].shape)).astype(np.float32)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], SMALL_CU,
                          inp["h0"], do, dht, 1.0, kda=True)
    got = run_bwd(inp, do, dht, 1.0)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert bool(torch.isfinite(got[key][:SMALL_CU[-1]]).all()), key
    errs = compare(inp, got, ref)
    _say("bwd kda strong decay: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_backward_kda_mixed_block_decay():
    """KDA gates where only rows 16..31 of every chunk decay steeply in one
    channel (g = -5 there: the block's last row is e^-75 from its first):
    that 16-row block takes the pair-by-pair sums in the prep and the final
    pass, the chunk's other blocks the factored MFMA products, in the same
    cell.  Every gradient must match the oracle."""
    inp = make_inputs(SMALL_CU[-1], 2, 64, 64, kda=True, dtype="bf16", seed=790,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    cu = np.asarray(SMALL_CU)
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            if 16 <= (t - cu[n]) % 64 < 32:
                inp["g"][t, :, 5] = -5.0
    rng = np.random.default_rng(791)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    ref = gated_delta_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], SMALL_CU,
                          inp["h0"], do, dht, 1.0, kda=True)
    got = run_bwd(inp, do, dht, 1.0)
    errs = compare(inp, got, ref)
    _say("bwd kda mixed block decay: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs


def test_backward_concurrent_streams_match_sequential():
    """Two host threads issue backward calls on two streams at once, each
    forking its reverse pass onto its own second stream with its own events:
    every output must equal the same call run alone on one stream."""
    import threading
    cases = []
    for seed in (790, 791):
        inp = make_inputs(SMALL_CU[-1], 2, 64, 64, kda=False, dtype="bf16", seed=seed,
                          cu_seqlens=SMALL_CU, h0_std=0.1)
        rng = np.random.default_rng(seed + 1)
        do = rng.standard_normal(inp["v"].shape).astype(np.float32)
        dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
        cases.append((inp, do, dht))
    alone = [run_bwd(inp, do, dht, 1.0) for inp, do, dht in cases]

    def prepared(inp, do, dht):
        d = {x: torch.from_numpy(inp[x]).cuda().to(torch.bfloat16).contiguous() for x in ("q", "k", "v")}
        cu = torch.tensor(SMALL_CU, dtype=torch.int32, device="cuda")
        ci, co, _ = la.build_chunk_meta(cu, inp["q"].shape[0])
        return dict(q=d["q"], k=d["k"], v=d["v"], g=torch.from_numpy(inp["g"]).cuda(),
                    beta=torch.from_numpy(inp["beta"]).cuda(), cu=cu, ci=ci, co=co,
                    h0=torch.from_numpy(inp["h0"]).cuda(), do=torch.from_numpy(do).cuda(),
                    dht=torch.from_numpy(dht).cuda())

    args = [prepared(*c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    aux = [torch.cuda.Stream(), torch.cuda.Stream()]
    events = [la.fork_join_events(), la.fork_join_events()]
    torch.cuda.synchronize()
    results = [[None] * 4, [None] * 4]
    start = threading.Barrier(2)

    def worker(i):
        a = args[i]
        start.wait()
        with torch.cuda.stream(streams[i]):
            for rep in range(4):
                results[i][rep] = la.gdn_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"],
                                                   a["ci"], a["co"], a["do"], h0=a["h0"], dht=a["dht"],
                                                   scale=1.0, aux_stream=aux[i], events=events[i])
        streams[i].synchronize()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)
    for i in range(2):
        for rep in range(4):
            got = dict(zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), results[i][rep]))
            for key in ("dq", "dk", "dv", "dg", "dbeta"):
                assert torch.equal(got[key][:SMALL_CU[-1]], alone[i][key][:SMALL_CU[-1]]), (i, rep, key)
            assert torch.equal(got["dh0"][ne], alone[i]["dh0"][ne]), (i, rep)


def test_backward_default_allocations_fill_padding():
    """Outputs the binding allocates: rows outside every sequence are zero,
    dh0 of a zero-length sequence is its dht (the state passes through
    unchanged), and every value is finite."""
    inp = make_inputs(SMALL_CU[-1] + 37, 2, 64, 64, kda=False, dtype="bf16", seed=795,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    rng = np.random.default_rng(796)
    do = rng.standard_normal(inp["v"].shape).astype(np.float32)
    dht = rng.standard_normal(inp["h0"].shape).astype(np.float32)
    got = run_bwd(inp, do, dht, 1.0)
    rows = SMALL_CU[-1]
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        t = got[key]
        assert bool(torch.isfinite(t).all()), key
        assert bool((t[rows:] == 0).all()), key
    empty = np.flatnonzero(np.diff(np.asarray(SMALL_CU)) == 0)
    assert len(empty) > 0
    for n in empty:
        assert torch.equal(got["dh0"][n].cpu(), torch.from_numpy(dht[n])), n
