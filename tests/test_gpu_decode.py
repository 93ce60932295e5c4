"""GPU parity of the recurrent (decode) step: one token per sequence, the
state updated in place, against the fp64 oracle's token recurrence on
sequences of length one (the same definition the chunk forward follows).

Bar: max relative error <= 2e-3 (bf16 inputs) / 1e-4 (fp32 inputs); the
step computes in fp32 throughout, so the measured errors are far below.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from synth import make_inputs
from tests.helpers import TOL, TORCH_DT, gva, rel_err, rel_err_bf16_out, run_oracle

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _step_inputs(N, H, d, kda, dtype, seed, h0_std=0.1):
    """N one-token sequences (cu_seqlens = 0, 1, .., N) from the shared
    generator: token n of the batch is sequence n."""
    return make_inputs(N, H, d, d, kda=kda, dtype=dtype, seed=seed,
                       cu_seqlens=np.arange(N + 1, dtype=np.int32), h0_std=h0_std)


def _dev(inp):
    tdt = TORCH_DT[inp["dtype"]]
    d = {key: torch.from_numpy(inp[key]).cuda().to(tdt).contiguous() for key in ("q", "k", "v")}
    for key in ("g", "beta"):
        d[key] = torch.from_numpy(inp[key]).cuda().contiguous()
    d["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).cuda().contiguous()
    return d


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 128),
                                     ("f32", 64)])
def test_recurrent_step_matches_oracle(kda, dtype, d):
    inp = _step_inputs(37, 5, d, kda, dtype, seed=200 + d)
    dv = _dev(inp)
    fwd = la.kda_recurrent_fwd if kda else la.gdn_recurrent_fwd
    o, ht = fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], h0=dv["h0"], scale=0.7)
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(inp, scale=0.7)
    eo = rel_err(o.cpu().numpy(), o_ref)
    eh = rel_err(ht.cpu().numpy(), ht_ref)
    _say(f"decode kda={kda} {dtype} d={d}: o {eo:.2e} ht {eh:.2e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_recurrent_steps_in_place_match_prefill(kda):
    """Eight decode steps in place (ht = h0) equal the oracle over the
    8-token sequences; the state buffer is the only carrier."""
    N, H, d, steps = 6, 3, 128, 8
    inp = make_inputs(N * steps, H, d, d, kda=kda, dtype="bf16", seed=210,
                      cu_seqlens=np.arange(0, N * steps + 1, steps, dtype=np.int32), h0_std=0.1)
    state = torch.from_numpy(inp["h0"]).cuda().contiguous()
    fwd = la.kda_recurrent_fwd if kda else la.gdn_recurrent_fwd
    outs = []
    for t in range(steps):
        rows = np.arange(N) * steps + t  # token t of every sequence
        sel = {key: torch.from_numpy(np.ascontiguousarray(inp[key][rows])).cuda()
               for key in ("q", "k", "v", "g", "beta")}
        for key in ("q", "k", "v"):
            sel[key] = sel[key].to(torch.bfloat16)
        o, ht = fwd(sel["q"], sel["k"], sel["v"], sel["g"], sel["beta"], h0=state, ht=state)
        assert ht.data_ptr() == state.data_ptr()
        outs.append(o.cpu().numpy())
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(inp)
    o_dec = np.stack(outs, axis=1).reshape(N * steps, H, d)
    eo = rel_err(o_dec, o_ref)
    eh = rel_err(state.cpu().numpy(), ht_ref)
    _say(f"decode x{steps} in place kda={kda}: o {eo:.2e} ht {eh:.2e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_recurrent_zero_state_and_no_final_state():
    """h0 = NULL is the zero state; ht = NULL writes no state."""
    inp = _step_inputs(9, 4, 64, False, "bf16", seed=220, h0_std=None)
    dv = _dev(inp)
    o, ht = la.gdn_recurrent_fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"],
                                 output_final_state=False)
    torch.cuda.synchronize()
    assert ht is None
    o_ref, _ = run_oracle(inp)
    eo = rel_err(o.cpu().numpy(), o_ref)
    _say(f"decode zero state: o {eo:.2e}")
    assert eo <= TOL["bf16"]


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_recurrent_grouped_value_heads_and_bf16_output(kda):
    """8 value heads over 2 q/k heads; o in bf16 equals the rounded fp32 o."""
    inp = _step_inputs(21, 8, 128, kda, "bf16", seed=230)
    small, full = gva(inp, 2)
    dv = _dev(small)
    fwd = la.kda_recurrent_fwd if kda else la.gdn_recurrent_fwd
    o, ht = fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], h0=dv["h0"])
    o16, _ = fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], h0=dv["h0"],
                 o_dtype=torch.bfloat16, output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o16, o.to(torch.bfloat16))
    o_ref, ht_ref = run_oracle(full)
    eo = rel_err(o.cpu().numpy(), o_ref)
    eh = rel_err(ht.cpu().numpy(), ht_ref)
    e16 = rel_err_bf16_out(o16.float().cpu().numpy(), o_ref)
    _say(f"decode GVA + bf16 o kda={kda}: o {eo:.2e} ht {eh:.2e} bf16 o {e16:.2e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"] and e16 <= TOL["bf16"]


@pytest.mark.parametrize("i", range(24))
def test_recurrent_random_shapes(i):
    """Seeded random decode batches: GDN or KDA, bf16 / fp16 / fp32, d = 64
    or 128, 1 to 200 sequences, 1 to 16 heads, with or without h0, against
    the oracle's token recurrence."""
    rng = np.random.default_rng(60_000 + i)
    kda = bool(rng.integers(2))
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    d = int(rng.choice([64, 128]))
    N, H = int(rng.integers(1, 201)), int(rng.integers(1, 17))
    h0_std = 0.1 if rng.random() < 0.8 else None
    scale = float(rng.choice([1.0, d ** -0.5]))
    inp = _step_inputs(N, H, d, kda, dtype, seed=int(rng.integers(1 << 30)), h0_std=h0_std)
    dv = _dev(inp)
    fwd = la.kda_recurrent_fwd if kda else la.gdn_recurrent_fwd
    o, ht = fwd(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], h0=dv["h0"], scale=scale)
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(inp, scale=scale)
    eo = rel_err(o.cpu().numpy(), o_ref)
    eh = rel_err(ht.cpu().numpy(), ht_ref)
    _say(f"decode random {i}: kda={kda} {dtype} d={d} N={N} H={H} h0={h0_std is not None}: "
         f"o {eo:.2e} ht {eh:.2e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
