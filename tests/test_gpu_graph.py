"""Graph capture and replay over a fixed-capacity bucket.

The FLA graph-capture RFC (sections "Proposed design" and "Test plan") asks
for: metadata built on the device from a fixed-shape cu_seqlens, one capture
of a fixed grid sized by NT_max and N_max, then replays after copying fresh
cu_seqlens and inputs into the same static buffers; replays must equal the
eager call on the same buffers bit for bit, padding must not leak, and
unused slots must not be written.  Each replay here is checked bitwise
against an eager call on the same buffers and against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from synth import bucket_layout, config, make_inputs
from tests.helpers import compare, run_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


class Bucket:
    """Static device buffers of one bucket and the captured step."""

    def __init__(self, T_max, N_max, H, d, kda, with_h0):
        dev = torch.device("cuda")
        self.kda, self.T_max, self.N_max = kda, T_max, N_max
        bf = torch.bfloat16
        self.q = torch.zeros((T_max, H, d), dtype=bf, device=dev)
        self.k = torch.zeros_like(self.q)
        self.v = torch.zeros_like(self.q)
        self.g = torch.zeros((T_max, H, d) if kda else (T_max, H), device=dev)
        self.beta = torch.zeros((T_max, H), device=dev)
        self.cu = torch.zeros((N_max + 1,), dtype=torch.int32, device=dev)
        NT = la.nt_max(T_max, N_max)
        self.ci = torch.empty((NT, 2), dtype=torch.int32, device=dev)
        self.co = torch.empty((N_max + 1,), dtype=torch.int32, device=dev)
        self.st = torch.empty((1,), dtype=torch.int32, device=dev)
        self.h0 = torch.zeros((N_max, H, d, d), device=dev) if with_h0 else None
        self.o = torch.empty((T_max, H, d), device=dev)
        self.ht = torch.empty((N_max, H, d, d), device=dev)
        self.ws = torch.empty((la.workspace_bytes(T_max, N_max, H, d, d, bf, kda),),
                              dtype=torch.uint8, device=dev)
        self.graph = None

    def fill(self, inp):
        """Copy a layout and its inputs into the static buffers (outside the graph)."""
        for name in ("q", "k", "v"):
            getattr(self, name).copy_(torch.from_numpy(inp[name]).to(torch.bfloat16))
        self.g.copy_(torch.from_numpy(inp["g"]))
        self.beta.copy_(torch.from_numpy(inp["beta"]))
        self.cu.copy_(torch.from_numpy(inp["cu_seqlens"].astype(np.int32)))
        if self.h0 is not None:
            self.h0.copy_(torch.from_numpy(inp["h0"]))

    def step(self):
        la.build_chunk_meta(self.cu, self.T_max, chunk_indices=self.ci, chunk_offsets=self.co,
                            status=self.st)
        fwd = la.kda_chunk_fwd if self.kda else la.gdn_chunk_fwd
        fwd(self.q, self.k, self.v, self.g, self.beta, self.cu, self.ci, self.co, h0=self.h0,
            o=self.o, ht=self.ht, workspace=self.ws)

    def capture(self):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()
        torch.cuda.synchronize()


def _canary(b):
    b.o.fill_(321.0)
    b.ht.fill_(-9.0)


def _check_replay(b, inp, heads, label):
    """Replay, then eager on the same buffers: bitwise equal; oracle parity on
    ``heads``; padding rows and empty-sequence states keep their canaries."""
    cu = inp["cu_seqlens"]
    total = int(cu[-1])
    _canary(b)
    b.graph.replay()
    torch.cuda.synchronize()
    assert int(b.st.item()) == 0
    o_g, ht_g = b.o.clone(), b.ht.clone()
    # the same buffers through the eager path
    _canary(b)
    b.step()
    torch.cuda.synchronize()
    assert torch.equal(b.o, o_g), f"{label}: graph o != eager o"
    assert torch.equal(b.ht, ht_g), f"{label}: graph ht != eager ht"
    o_np, ht_np = o_g.cpu().numpy(), ht_g.cpu().numpy()
    assert (o_np[total:] == 321.0).all(), f"{label}: padding rows written"
    empty = np.diff(cu.astype(np.int64)) == 0
    assert (ht_np[empty] == -9.0).all(), f"{label}: empty-sequence state written"
    o_ref, ht_ref = run_oracle(inp, heads=heads)
    eo, eh, tol = compare(inp, o_g, ht_g, o_ref, ht_ref, heads=heads)
    _say(f"{label}: N={int((~empty).sum())} total={total} o {eo:.2e} ht {eh:.2e}")
    assert eo <= tol and eh <= tol
    return o_g, ht_g


def test_bucket_graph_replays_fresh_layouts():
    """The fixed-capacity bucket: T_max=16384, N_max=64, GDN bf16, H=32, d=128,
    no initial state; one capture, fresh layout and inputs per replay."""
    b = Bucket(16384, 64, 32, 128, kda=False, with_h0=False)
    b.fill(config(3, replay=0))
    b.capture()
    for r in range(3):
        inp = config(3, replay=r)
        b.fill(inp)
        _check_replay(b, inp, heads=[r, 31 - r], label=f"bucket replay {r}")


def test_graph_replays_are_stable_with_eager_work_between():
    """Several replays of one layout, with unrelated eager work and
    synchronisations in between, all bitwise equal to the eager result."""
    cu = [0, 700, 700, 1500, 1501, 2000]
    inp = make_inputs(2048, 4, 128, 128, kda=False, dtype="bf16", seed=61, cu_seqlens=cu,
                      h0_std=0.1)
    b = Bucket(2048, 5, 4, 128, kda=False, with_h0=True)
    b.fill(inp)
    b.capture()
    b.step()
    torch.cuda.synchronize()
    o_e, ht_e = b.o.clone(), b.ht.clone()
    x = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        b.graph.replay()
        y = (x * (i + 1)).sum()          # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(y)
        assert torch.equal(b.o, o_e) and torch.equal(b.ht, ht_e), f"replay {i} differs"


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_small_bucket_graph_layouts_with_state(kda):
    """A small bucket with initial states: layouts with empty, one-token and
    exact-chunk sequences, NaN in the padding rows of one replay."""
    T_max, N_max, H, d = 1536, 8, 3, 128
    b = Bucket(T_max, N_max, H, d, kda=kda, with_h0=True)
    rng = np.random.default_rng(62)
    layouts = [bucket_layout(rng, T_max, N_max),
               np.array([0, 1, 1, 65, 129, 129, 700, 1000, 1000], dtype=np.int32),
               bucket_layout(rng, 900, N_max)]
    first = True
    for i, cu in enumerate(layouts):
        inp = make_inputs(T_max, H, d, d, kda=kda, dtype="bf16", seed=70 + i, cu_seqlens=cu,
                          h0_std=0.1)
        total = int(cu[-1])
        if i == 2:
            for key in ("q", "k", "v", "g", "beta"):
                inp[key][total:] = np.nan
        b.fill(inp)
        if first:
            b.capture()
            first = False
        o_g, ht_g = _check_replay(b, inp, heads=None, label=f"layout {i} kda={kda}")
        assert np.isfinite(o_g.cpu().numpy()[:total]).all()


@pytest.mark.parametrize("fork", [False, True], ids=["one_stream", "aux_stream"])
@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_backward_graph_replays_over_layouts(kda, fork):
    """The chunk backward under the same contract: metadata and backward
    captured once on static buffers, replayed over fresh layouts and inputs
    copied in; every replay equals an eager call on the same buffers bit for
    bit (rows of real tokens, dh0 of non-empty sequences).  With the caller's
    second stream and events, the capture holds the forked reverse pass."""
    T_max, N_max, H, d = 1024, 6, 2, 64
    dev = torch.device("cuda")
    bf = torch.bfloat16
    q = torch.zeros((T_max, H, d), dtype=bf, device=dev)
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    g = torch.zeros((T_max, H, d) if kda else (T_max, H), device=dev)
    beta = torch.zeros((T_max, H), device=dev)
    cu = torch.zeros((N_max + 1,), dtype=torch.int32, device=dev)
    NT = la.nt_max(T_max, N_max)
    ci = torch.empty((NT, 2), dtype=torch.int32, device=dev)
    co = torch.empty((N_max + 1,), dtype=torch.int32, device=dev)
    h0 = torch.zeros((N_max, H, d, d), device=dev)
    dout = torch.zeros((T_max, H, d), device=dev)
    outs = dict(dq=torch.zeros((T_max, H, d), device=dev), dk=torch.zeros((T_max, H, d), device=dev),
                dv=torch.zeros((T_max, H, d), device=dev), dg=torch.zeros(g.shape, device=dev),
                dbeta=torch.zeros((T_max, H), device=dev), dh0=torch.zeros_like(h0))
    ws = torch.empty((la.bwd_workspace_bytes(T_max, N_max, H, d, d, bf, kda=kda),),
                     dtype=torch.uint8, device=dev)
    fn = la.kda_chunk_bwd if kda else la.gdn_chunk_bwd
    side = dict(aux_stream=torch.cuda.Stream(), events=la.fork_join_events()) if fork else {}

    def step():
        la.build_chunk_meta(cu, T_max, chunk_indices=ci, chunk_offsets=co)
        fn(q, k, v, g, beta, cu, ci, co, dout, h0=h0, workspace=ws, **outs, **side)

    def fill(seed):
        rng = np.random.default_rng(seed)
        lay = bucket_layout(rng, T_max, N_max)
        inp = make_inputs(T_max, H, d, d, kda=kda, dtype="bf16", seed=seed, cu_seqlens=lay,
                          h0_std=0.1)
        q.copy_(torch.from_numpy(inp["q"]).to(bf))
        k.copy_(torch.from_numpy(inp["k"]).to(bf))
        v.copy_(torch.from_numpy(inp["v"]).to(bf))
        g.copy_(torch.from_numpy(inp["g"]))
        beta.copy_(torch.from_numpy(inp["beta"]))
        cu.copy_(torch.from_numpy(lay.astype(np.int32)))
        h0.copy_(torch.from_numpy(inp["h0"]))
        dout.copy_(torch.from_numpy(rng.standard_normal((T_max, H, d)).astype(np.float32)))
        return lay

    fill(900)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        lay = fill(901 + r)
        step()
        torch.cuda.synchronize()
        eager = {key: t.clone() for key, t in outs.items()}
        graph.replay()
        torch.cuda.synchronize()
        rows = int(lay[-1])
        ne = torch.from_numpy(np.diff(lay) > 0)
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(outs[key][:rows], eager[key][:rows]), (r, key)
        assert torch.equal(outs["dh0"][ne], eager["dh0"][ne]), r
        _say(f"backward graph replay {r} (fork {fork}): {int((np.diff(lay) > 0).sum())} "
             f"sequences, {rows} tokens")


def test_short_conv_graph_replays_over_layouts():
    """The short convolution captured once with the metadata and replayed over
    fresh layouts, states updated in place: each replay equals an eager call."""
    T_max, N_max, D, W = 1024, 6, 512, 4
    dev = torch.device("cuda")
    bf = torch.bfloat16
    x = torch.zeros((T_max, D), dtype=bf, device=dev)
    w = torch.zeros((D, W), device=dev)
    b = torch.zeros((D,), device=dev)
    cu = torch.zeros((N_max + 1,), dtype=torch.int32, device=dev)
    NT = la.nt_max(T_max, N_max)
    ci = torch.empty((NT, 2), dtype=torch.int32, device=dev)
    co = torch.empty((N_max + 1,), dtype=torch.int32, device=dev)
    state = torch.zeros((N_max, W - 1, D), dtype=bf, device=dev)
    y = torch.zeros((T_max, D), dtype=bf, device=dev)

    def step():
        la.build_chunk_meta(cu, T_max, chunk_indices=ci, chunk_offsets=co)
        la.short_conv_fwd(x, w, cu, ci, bias=b, h0=state, ht=state, y=y, activation="silu")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    from synth import make_conv_inputs
    for r in range(4):
        rng = np.random.default_rng(950 + r)
        lay = bucket_layout(rng, T_max, N_max)
        inp = make_conv_inputs(T_max, D, W, dtype="bf16", seed=950 + r, cu_seqlens=lay, h0=True)
        x.copy_(torch.from_numpy(inp["x"]).to(bf))
        w.copy_(torch.from_numpy(inp["weight"]))
        b.copy_(torch.from_numpy(inp["bias"]))
        cu.copy_(torch.from_numpy(lay.astype(np.int32)))
        s0 = torch.from_numpy(inp["h0"]).to(dev, bf)
        state.copy_(s0)
        step()
        torch.cuda.synchronize()
        ey, es = y.clone(), state.clone()
        state.copy_(s0)
        graph.replay()
        torch.cuda.synchronize()
        rows = int(lay[-1])
        ne = torch.from_numpy(np.diff(lay) > 0)
        assert torch.equal(y[:rows], ey[:rows]) and torch.equal(state[ne], es[ne]), r
