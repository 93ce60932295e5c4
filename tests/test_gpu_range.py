"""GPU parity of the chunk forward over the input scale.

bf16 and fp16 inputs run on fp16 MFMA operands, whose exponent range is
narrower than bf16's: tiny values fall onto fp16's subnormal grid and values
above 65504 overflow.  The recurrence is linear in (v, h0) jointly, so scaling
both by an exact power of two scales o and ht by the same factor; the oracle
sees the scaled values.  The reduce runs each wave's state-side operands
times a power of two chosen from the initial state and the first chunk's v,
so these cases, 2^-24 to 2^16, all meet the bf16 gate
(max |x - ref| / max |ref| <= 2e-3), GDN and KDA, one-pass and segmented.
"""

import numpy as np
import pytest

from synth import make_inputs
from tests.helpers import TOL, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

CU = [0, 1, 70, 70, 200, 457]


@pytest.mark.parametrize("seg", [-1, 2], ids=["one_pass", "segmented"])
@pytest.mark.parametrize("log2_scale", [-24, -16, -12, 8, 16])
@pytest.mark.parametrize("kda", [False, True], ids=["gdn", "kda"])
def test_forward_input_scale(kda, log2_scale, seg):
    inp = make_inputs(CU[-1], 2, 128, 128, kda=kda, dtype="bf16", seed=950 + log2_scale,
                      cu_seqlens=CU, h0_std=0.1)
    s = np.float32(2.0 ** log2_scale)
    inp["v"] = inp["v"] * s          # exact: a power of two on bf16 values
    inp["h0"] = inp["h0"] * s
    o, ht, _ = run_gpu(inp, seg_len=seg)
    o_ref, ht_ref = run_oracle(inp)
    eo, eh, tol = compare(inp, o, ht, o_ref, ht_ref)
    print(f"scale 2^{log2_scale} kda={kda} seg={seg}: o {eo:.2e} ht {eh:.2e}", flush=True)
    assert np.isfinite(o.cpu().numpy()[:CU[-1]]).all()
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]
