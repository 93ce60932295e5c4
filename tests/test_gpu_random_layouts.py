"""GPU: the forward on seeded random varlen layouts, against the oracle.

Each case draws its own shape and options from a seeded generator: GDN or
KDA; bf16, fp16 or fp32 inputs (d = 64 or 128; fp32 at 64); 1 to 6 heads;
1 to 69 sequences whose lengths mix empty, one-token, exact multiples of the
64-row chunk and arbitrary lengths up to 299; with or without an initial
state; automatic or forced state-column slices; the one-pass, the forced
one-pass or a 4-chunk segmented reduce (16-bit inputs); and the layout from
build_chunk_meta or built by the call itself.  o over the real rows and ht
over non-empty sequences must meet the dtype's tolerance.  A combination the
boundary rejects must raise LinAttnError, never launch.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from synth import make_inputs
from tests.helpers import TOL, compare, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(90_000 + i)
    kda = bool(rng.integers(2))
    dt = ["bf16", "f16", "f32"][rng.integers(3)]
    d = 64 if dt == "f32" else int(rng.choice([64, 128]))
    H = int(rng.integers(1, 7))
    N = int(rng.integers(1, 70))
    lens = rng.integers(0, 300, N)
    lens[rng.random(N) < 0.15] = 0
    lens[rng.random(N) < 0.1] = 1
    lens[rng.random(N) < 0.1] = 64 * int(rng.integers(1, 4))
    if lens.sum() == 0:
        lens[0] = 5
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    h0 = 0.1 if rng.random() < 0.7 else None
    split = int(rng.choice([0, 0, 1, 2, 4])) if d == 128 else int(rng.choice([0, 1, 2]))
    if d // max(split, 1) < 32:
        split = 0
    seg = int(rng.choice([0, 0, -1, 4])) if dt != "f32" and N <= 64 else 0
    build = dt != "f32" and bool(rng.random() < 0.5)
    inp = make_inputs(int(cu[-1]), H, d, d, kda=kda, dtype=dt, seed=int(rng.integers(1 << 30)),
                      cu_seqlens=cu, h0_std=h0)
    return inp, split, seg, build


@pytest.mark.parametrize("i", range(60))
def test_random_layout(i):
    inp, split, seg, build = _case(i)
    T, N = inp["q"].shape[0], len(inp["cu_seqlens"]) - 1
    print(f"random layout {i}: kda={inp['kda']} {inp['dtype']} d={inp['dk']} H={inp['H']} "
          f"N={N} T={T} split={split} seg={seg} build={build}", flush=True)
    try:
        if build:
            dv = to_dev(inp)
            ci = torch.full((la.nt_max(T, N), 2), -7, dtype=torch.int32, device="cuda")
            co = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
            f = la.kda_chunk_fwd if inp["kda"] else la.gdn_chunk_fwd
            o, ht = f(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["cu_seqlens"], ci, co,
                      h0=dv["h0"], dv_split=split, seg_len=seg, build_meta=True)
            torch.cuda.synchronize()
        else:
            o, ht, _ = run_gpu(inp, dv_split=split, seg_len=seg)
    except la.LinAttnError:
        pytest.skip("combination rejected by the boundary")
    o_ref, ht_ref = run_oracle(inp)
    eo, eh, tol = compare(inp, o, ht, o_ref, ht_ref)
    print(f"   o {eo:.2e} ht {eh:.2e}", flush=True)
    assert np.isfinite(eo) and np.isfinite(eh)
    assert eo <= tol and eh <= tol
