"""GPU parity of the test-matrix variants the graph-capture RFC lists for
every operator (section "Testing"): fp16 inputs, int64 cu_seqlens and
BT = 32 layouts (the metadata itself, and the forward and backward given
BT = 32 metadata).

Bar: as for the bf16 path (max relative error <= 2e-3 against the fp64
oracle; fp16 inputs use the same fp16 MFMA operands); metadata bit-exact
against the oracle's; int64 and int32 cu_seqlens give bit-identical outputs.
"""

import numpy as np
import pytest
import torch

import chunkwise_gated_delta_chunk_amd as la
from oracle import meta_ref
from synth import bucket_layout, make_inputs
from tests.helpers import compare, rel_err_bf16_out, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu

SMALL_CU = [0, 1, 64, 64, 200, 333, 460]   # one-token, exact chunk, empty, tails


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------- fp16 inputs ---
@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp16_inputs(kda, d):
    inp = make_inputs(SMALL_CU[-1], 3, d, d, kda=kda, dtype="f16", seed=300 + d,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    o_ref, ht_ref = run_oracle(inp)
    for split in (0, 1, d // 32):
        o, ht, _ = run_gpu(inp, dv_split=split)
        eo, eh, tol = compare(inp, o, ht, o_ref, ht_ref)
        _say(f"fp16 kda={kda} d={d} split={split}: o {eo:.2e} ht {eh:.2e}")
        assert eo <= tol and eh <= tol


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_fp16_segmented_and_bf16_output(kda):
    cu = [0, 700, 710, 1500]
    inp = make_inputs(cu[-1], 2, 128, 128, kda=kda, dtype="f16", seed=310, cu_seqlens=cu,
                      h0_std=0.1)
    o_ref, ht_ref = run_oracle(inp)
    o, ht, _ = run_gpu(inp, seg_len=3)
    eo, eh, tol = compare(inp, o, ht, o_ref, ht_ref)
    _say(f"fp16 segmented kda={kda}: o {eo:.2e} ht {eh:.2e}")
    assert eo <= tol and eh <= tol
    ob, htb, _ = run_gpu(inp, o_dtype=torch.bfloat16)
    assert ob.dtype == torch.bfloat16
    eo = rel_err_bf16_out(ob.float().cpu().numpy(), o_ref)
    _say(f"fp16 in, bf16 out kda={kda}: o {eo:.2e}")
    assert eo <= tol


def test_fp16_matches_bf16_path_on_shared_values():
    """Inputs representable in both formats (bf16 values within fp16's normal
    range with at most 8 significant bits) give the same result either way:
    both paths feed the same fp16 operands to the same kernels."""
    inp = make_inputs(SMALL_CU[-1], 2, 128, 128, kda=False, dtype="bf16", seed=320,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    for x in ("q", "k", "v"):   # keep away from fp16 subnormals
        a = inp[x]
        inp[x] = np.where(np.abs(a) < 2.0 ** -14, 0.0, a).astype(np.float32)
    o1, h1, _ = run_gpu(inp)
    inp16 = dict(inp, dtype="f16")
    o2, h2, _ = run_gpu(inp16)
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)   # ht of empty sequences: unwritten
    assert torch.equal(o1, o2) and torch.equal(h1[ne], h2[ne])


# ------------------------------------------------------ int64 cu_seqlens ---
@pytest.mark.parametrize("BT", [32, 64])
@pytest.mark.parametrize("seed", range(3))
def test_meta_int64_and_bt32_random_layouts(BT, seed):
    rng = np.random.default_rng(500 + seed)
    for _ in range(8):
        T_max = int(rng.integers(1, 20000))
        N_max = int(rng.integers(1, 300))
        cu = bucket_layout(rng, T_max, N_max).tolist()
        ref = meta_ref.chunk_meta(cu, N_max, T_max, BT)
        for idx in (torch.int32, torch.int64):
            ci, co, st = la.build_chunk_meta(torch.tensor(cu, dtype=idx, device="cuda"), T_max, BT)
            torch.cuda.synchronize()
            assert np.array_equal(ci.cpu().numpy(), ref[0])
            assert np.array_equal(co.cpu().numpy(), ref[1])
            assert int(st.item()) == ref[2]


def test_meta_int64_values_beyond_int32():
    """Offsets that only an int64 check sees as invalid: truncated to 32 bits
    they would look like a valid layout."""
    big = 1 << 32
    cases = [
        ([0, big + 10, big + 20], 100),          # low words 10, 20: valid if truncated
        ([0, 10, big + 5, 30], 100),
        ([0, -big + 5, 50], 100),                # low word 5
        ([big, big + 10], 100),                  # cu[0] low word 0
    ]
    for cu, T_max in cases:
        N_max = len(cu) - 1
        ref_i, ref_o, ref_s = meta_ref.chunk_meta(cu, N_max, T_max, 64)
        assert ref_s != 0
        ci, co, st = la.build_chunk_meta(torch.tensor(cu, dtype=torch.int64, device="cuda"), T_max)
        torch.cuda.synchronize()
        _say("int64 case", cu, "status", int(st.item()), "oracle", ref_s)
        assert int(st.item()) == ref_s
        assert np.array_equal(ci.cpu().numpy(), ref_i)
        assert np.array_equal(co.cpu().numpy(), ref_o)


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_forward_int64_cu_seqlens(kda):
    inp = make_inputs(SMALL_CU[-1], 3, 128, 128, kda=kda, dtype="bf16", seed=330,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    o32, h32, _ = run_gpu(inp)
    o64, h64, (ci, co, st) = run_gpu(inp, cu_dtype=torch.int64)
    assert int(st.item()) == 0
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)   # ht of empty sequences: unwritten
    assert torch.equal(o32, o64) and torch.equal(h32[ne], h64[ne])
    o_ref, ht_ref = run_oracle(inp)
    eo, eh, tol = compare(inp, o64, h64, o_ref, ht_ref)
    _say(f"int64 cu kda={kda}: o {eo:.2e} ht {eh:.2e}")
    assert eo <= tol and eh <= tol
    # segmented reduce reads the offsets too
    o64s, h64s, _ = run_gpu(inp, cu_dtype=torch.int64, seg_len=2)
    eo, eh, tol = compare(inp, o64s, h64s, o_ref, ht_ref)
    assert eo <= tol and eh <= tol


def test_forward_int64_invalid_writes_nothing():
    cu = [0, (1 << 32) + 100, (1 << 32) + 200]
    inp = make_inputs(256, 2, 64, 64, kda=False, dtype="bf16", seed=340, cu_seqlens=[0, 100, 200])
    d = to_dev(inp)
    cu_t = torch.tensor(cu, dtype=torch.int64, device="cuda")
    ci, co, st = la.build_chunk_meta(cu_t, 256)
    o = torch.full((256, 2, 64), 7.0, device="cuda")
    ht = torch.full((2, 2, 64, 64), 5.0, device="cuda")
    la.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_t, ci, co, o=o, ht=ht)
    torch.cuda.synchronize()
    assert int(st.item()) != 0
    assert bool((o == 7.0).all()) and bool((ht == 5.0).all())


# ------------------------------------------------------------- BT = 32 ---
@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
@pytest.mark.parametrize("seg", [-1, 2])
def test_forward_with_bt32_layout(kda, seg):
    """A caller's BT = 32 metadata: the call rebuilds the 64-row layout its
    kernels run on from cu_seqlens, so the result equals the BT = 64 call bit
    for bit, and the oracle within the gate."""
    inp = make_inputs(SMALL_CU[-1], 2, 128, 128, kda=kda, dtype="bf16", seed=350,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    d = to_dev(inp)
    T = SMALL_CU[-1]
    fwd = la.kda_chunk_fwd if kda else la.gdn_chunk_fwd
    res = {}
    for BT in (64, 32):
        ci, co, st = la.build_chunk_meta(d["cu_seqlens"], T, BT)
        o, ht = fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ci, co,
                    h0=d["h0"], seg_len=seg, BT=BT)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        res[BT] = (o, ht)
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)
    assert torch.equal(res[32][0][:T], res[64][0][:T])
    assert torch.equal(res[32][1][ne], res[64][1][ne])
    o_ref, ht_ref = run_oracle(inp)
    eo, eh, tol = compare(inp, res[32][0], res[32][1], o_ref, ht_ref)
    _say(f"BT=32 layout kda={kda} seg={seg}: o {eo:.2e} ht {eh:.2e}")
    assert eo <= tol and eh <= tol


@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_backward_with_bt32_layout(kda):
    inp = make_inputs(SMALL_CU[-1], 2, 64, 64, kda=kda, dtype="bf16", seed=360,
                      cu_seqlens=SMALL_CU, h0_std=0.1)
    d = to_dev(inp)
    T = SMALL_CU[-1]
    rng = np.random.default_rng(361)
    dout = torch.from_numpy(rng.standard_normal(inp["v"].shape).astype(np.float32)).cuda()
    bwd = la.kda_chunk_bwd if kda else la.gdn_chunk_bwd
    res = {}
    for BT in (64, 32):
        ci, co, _ = la.build_chunk_meta(d["cu_seqlens"], T, BT)
        res[BT] = bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ci, co, dout,
                      h0=d["h0"], BT=BT)
        torch.cuda.synchronize()
    ne = torch.from_numpy(np.diff(np.asarray(SMALL_CU)) > 0)
    for i in range(5):
        assert torch.equal(res[32][i][:T], res[64][i][:T]), i
    assert torch.equal(res[32][5][ne], res[64][5][ne])
