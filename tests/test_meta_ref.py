"""Pins for the host metadata reference (CPU only): hand-computed layouts and
the capacity formula of the FLA graph-capture RFC, section "Fixed-capacity
execution", plus invariants over random layouts."""

import json
import os

import numpy as np
import pytest

from oracle import meta_ref
from synth import bucket_layout

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "meta_cases.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["name"] for c in GOLDEN["cases"]])
def test_hand_computed_layouts(case):
    idx, off, st = meta_ref.chunk_meta(case["cu"], case["N_max"], case["T_max"], case["BT"])
    assert meta_ref.nt_max(case["T_max"], case["N_max"], case["BT"]) == case["nt_max"]
    assert idx.shape == (case["nt_max"], 2)
    assert idx.tolist() == case["indices"]
    assert off.tolist() == case["offsets"]
    assert st == case["status"]


@pytest.mark.parametrize("c", GOLDEN["capacity"], ids=lambda c: f"{c['T_max']}-{c['N_max']}-{c['BT']}")
def test_capacity_formula(c):
    assert meta_ref.nt_max(c["T_max"], c["N_max"], c["BT"]) == c["nt_max"]


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("BT", [32, 64])
def test_random_layout_invariants(seed, BT):
    rng = np.random.default_rng(seed)
    T_max, N_max = int(rng.integers(1, 3000)), int(rng.integers(1, 70))
    cu = bucket_layout(rng, T_max, N_max)
    idx, off, st = meta_ref.chunk_meta(cu, N_max, T_max, BT)
    assert st == 0
    lens = np.diff(cu.astype(np.int64))
    nchunks = -(-lens // BT)
    used = int(nchunks.sum())
    assert used <= meta_ref.nt_max(T_max, N_max, BT)
    assert (idx[used:] == [-1, 0]).all()
    # every (n, i_t) with i_t < ceil(len_n/BT) appears exactly once, in order
    pairs = [(n, t) for n in range(N_max) for t in range(int(nchunks[n]))]
    assert [tuple(p) for p in idx[:used].tolist()] == pairs
    assert off[0] == 0 and (np.diff(off) == nchunks).all()


def test_bound_is_tight_with_worst_case_layout():
    # N_max - 1 one-token sequences plus one sequence holding the rest
    for T_max, N_max, BT in [(1000, 10, 64), (64, 3, 64), (257, 5, 32)]:
        cu = np.concatenate([np.arange(N_max), [T_max]]).astype(np.int32)
        idx, off, st = meta_ref.chunk_meta(cu, N_max, T_max, BT)
        used = int((idx[:, 0] >= 0).sum())
        assert used == (N_max - 1) + -(-(T_max - N_max + 1) // BT)
        assert used <= meta_ref.nt_max(T_max, N_max, BT)
