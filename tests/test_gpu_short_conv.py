"""GPU parity of the varlen causal short convolution against the fp64 oracle.

Bar: outputs are computed in fp32 and rounded once to the data type, so
every element must lie within half a unit in the last place of the oracle's
value (bf16 or fp16) plus 1e-5 of the largest |value| (the fp32 arithmetic);
fp32 outputs within 1e-5 relative to the largest |value|.  Final states are
copies of inputs and must be bit-exact.  Rows outside every sequence,
sentinel slots and the states of empty sequences are never written.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from oracle.short_conv import short_conv_fwd as conv_ref
from synth import make_conv_inputs
from tests.helpers import TORCH_DT

pytestmark = pytest.mark.gpu

GATE = 1e-5
CU = [0, 1, 3, 3, 70, 133, 200, 201]   # one token, shorter than W-1, empty, chunk spans


def _say(*a):
    print(*a, flush=True)


def _ulp(ref, dtype):
    a = np.abs(np.asarray(ref, dtype=np.float64))
    if dtype == "bf16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
        return np.exp2(e - 7)
    if dtype == "f16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return np.exp2(e - 10)
    return np.zeros_like(a)


def out_err(y, ref, dtype):
    """max over elements of (|y - ref| - half an ulp of ref) / max |ref|."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    over = np.maximum(np.abs(y - ref) - 0.5 * _ulp(ref, dtype), 0.0)
    return float(over.max() / max(np.abs(ref).max(), 1e-30))


def _dev(inp, idx=torch.int32):
    tdt = TORCH_DT[inp["dtype"]]
    d = {"x": torch.from_numpy(inp["x"]).cuda().to(tdt).contiguous(),
         "weight": torch.from_numpy(inp["weight"]).cuda().contiguous(),
         "cu": torch.from_numpy(inp["cu_seqlens"]).cuda().to(idx)}
    d["bias"] = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).cuda()
    d["residual"] = (None if inp["residual"] is None else
                     torch.from_numpy(inp["residual"]).cuda().to(tdt).contiguous())
    d["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).cuda().to(tdt).contiguous()
    return d


def run_conv(inp, *, BT=64, activation=None, idx=torch.int32, y=None, ht=None, h0="inp"):
    d = _dev(inp, idx)
    T = inp["x"].shape[0]
    ci, co, st = la.build_chunk_meta(d["cu"], T, BT)
    y, ht = la.short_conv_fwd(d["x"], d["weight"], d["cu"], ci, bias=d["bias"],
                              residual=d["residual"], h0=d["h0"] if h0 == "inp" else h0,
                              y=y, ht=ht, activation=activation, BT=BT)
    torch.cuda.synchronize()
    return y, ht


def check(inp, y, ht, activation, cu=None):
    cu = inp["cu_seqlens"] if cu is None else np.asarray(cu)
    y_ref, ht_ref = conv_ref(inp["x"], inp["weight"], cu, b=inp["bias"],
                             residual=inp["residual"], h0=inp["h0"], activation=activation)
    rows = int(cu[-1])
    ey = out_err(y.float().cpu().numpy()[:rows], y_ref[:rows], inp["dtype"])
    ok_h = True
    if ht is not None and inp["W"] > 1:
        ne = np.diff(cu) > 0
        got = ht.float().cpu().numpy()[ne]
        ok_h = np.array_equal(got, ht_ref[ne])
    return ey, ok_h


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("act", [None, "silu"])
def test_conv_matches_oracle(dtype, W, act):
    D = 1024 + 64 if dtype != "f32" else 520   # a ragged channel block
    inp = make_conv_inputs(CU[-1], D, W, dtype=dtype, seed=600 + W, cu_seqlens=CU,
                           residual=(W % 2 == 0), h0=True)
    for BT in (32, 64):
        y, ht = run_conv(inp, BT=BT, activation=act)
        ey, ok_h = check(inp, y, ht, act)
        _say(f"conv {dtype} W={W} act={act} BT={BT}: y {ey:.2e} ht exact {ok_h}")
        assert ey <= GATE and ok_h


def test_conv_no_bias_no_state():
    inp = make_conv_inputs(CU[-1], 512, 4, dtype="bf16", seed=610, cu_seqlens=CU, bias=False)
    y, ht = run_conv(inp, activation="silu")
    ey, ok_h = check(inp, y, ht, "silu")
    assert ey <= GATE and ok_h


def test_conv_in_place_state_and_two_part_replay():
    """ht == h0 updates the state in place; feeding a split batch part by part
    through the same state buffer gives the same outputs as one call, bit for
    bit (the partial-token replay case)."""
    T = 300
    cu_all = np.array([0, 140, 300])
    inp = make_conv_inputs(T, 512, 4, dtype="bf16", seed=620, cu_seqlens=cu_all,
                           residual=True, h0=True)
    y_all, ht_all = run_conv(inp, activation="silu")
    d = _dev(inp)
    state = d["h0"].clone()
    ys = []
    for a, b in ((0, 45), (45, 140)):   # sequence 0 in two parts, state in place
        x = d["x"][a:b].contiguous()
        r = d["residual"][a:b].contiguous()
        cu = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        ci, _, _ = la.build_chunk_meta(cu, b - a)
        s0 = state[0:1]
        y, _ = la.short_conv_fwd(x, d["weight"], cu, ci, bias=d["bias"], residual=r, h0=s0,
                                 ht=s0, activation="silu")
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys), y_all[:140])
    assert torch.equal(state[0], ht_all[0])


def test_conv_padding_sentinels_untouched_and_int64():
    T_max = 512
    cu = [0, 100, 100, 250]
    inp = make_conv_inputs(T_max, 512, 3, dtype="f16", seed=630, cu_seqlens=cu, h0=True)
    y0 = torch.full((T_max, 512), 3.0, dtype=torch.float16, device="cuda")
    h = torch.full((3, 2, 512), 5.0, dtype=torch.float16, device="cuda")
    y, ht = run_conv(inp, y=y0, ht=h, idx=torch.int64)
    assert bool((y[250:] == 3.0).all())
    assert bool((ht[1] == 5.0).all())            # empty sequence: not written
    ey, ok_h = check(inp, y, ht, None)
    assert ey <= GATE and ok_h


def test_conv_invalid_cu_writes_nothing():
    inp = make_conv_inputs(256, 512, 4, dtype="bf16", seed=640, cu_seqlens=[0, 200, 100])
    y0 = torch.full((256, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    y, _ = run_conv(inp, y=y0)
    assert bool((y == 3.0).all())


def test_conv_full_size_sampled_channels():
    """The benchmark's workload (T = 8192 in 8 sequences, D = 6144 bf16, W = 4,
    SiLU, states): channels are independent, so the oracle runs on a sample
    of 96 channels (two from each 128-channel group) and the rest is checked
    for finiteness."""
    from synth import config
    cu = config(1)["cu_seqlens"]
    inp = make_conv_inputs(8192, 6144, 4, dtype="bf16", seed=650, cu_seqlens=cu, h0=True)
    y, ht = run_conv(inp, activation="silu")
    cols = np.sort(np.concatenate([np.arange(0, 6144, 128), np.arange(127, 6144, 128)]))
    sub = dict(inp, x=inp["x"][:, cols], weight=inp["weight"][cols], bias=inp["bias"][cols],
               h0=inp["h0"][:, :, cols], D=len(cols))
    y_ref, ht_ref = conv_ref(sub["x"], sub["weight"], cu, b=sub["bias"], h0=sub["h0"],
                             activation="silu")
    ey = out_err(y.float().cpu().numpy()[:, cols], y_ref, "bf16")
    _say(f"conv full size sampled: y {ey:.2e}")
    assert ey <= GATE
    assert np.array_equal(ht.float().cpu().numpy()[:, :, cols], ht_ref)
    assert bool(torch.isfinite(y.float()).all())


@pytest.mark.parametrize("i", range(24))
def test_conv_random_layouts(i):
    """Seeded random varlen layouts (empty, one-token and longer sequences),
    channel counts (multiples of 8 for 16-bit x, of 4 for fp32), widths,
    BT, bias / residual / state and activation, against the oracle."""
    rng = np.random.default_rng(70_000 + i)
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    W = int(rng.integers(1, 5))
    D = int(rng.integers(1, 200)) * (8 if dtype != "f32" else 4)
    N = int(rng.integers(1, 40))
    lens = rng.integers(0, 150, N)
    lens[rng.random(N) < 0.2] = 0
    lens[rng.random(N) < 0.15] = 1
    if lens.sum() == 0:
        lens[0] = 3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    act = None if rng.random() < 0.5 else "silu"
    BT = int(rng.choice([32, 64]))
    inp = make_conv_inputs(int(cu[-1]), D, W, dtype=dtype, seed=int(rng.integers(1 << 30)),
                           cu_seqlens=cu, bias=bool(rng.random() < 0.7),
                           residual=bool(rng.random() < 0.5), h0=bool(rng.random() < 0.6))
    y, ht = run_conv(inp, BT=BT, activation=act)
    ey, ok_h = check(inp, y, ht, act)
    _say(f"conv random {i}: {dtype} W={W} D={D} N={N} T={int(cu[-1])} BT={BT} act={act}: "
         f"y {ey:.2e} ht exact {ok_h}")
    assert ey <= GATE and ok_h
