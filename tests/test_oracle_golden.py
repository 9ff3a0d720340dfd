"""Drift guard: the oracle still reproduces the sample stored by
tests/golden/make_golden.py (which calls only the oracle)."""
import json
import os

import numpy as np

import kda_inputs
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "oracle_w0_sample.json")


def test_oracle_reproduces_stored_sample():
    with open(GOLD) as f:
        ref = json.load(f)
    spec, cu, x = kda_inputs.workload(0)
    assert spec["name"] == ref["workload"]
    o, sf = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, eps=ref["eps"])
    np.testing.assert_allclose(o.reshape(-1)[ref["o_flat_index"]], ref["o_values"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sf.sum(), ref["final_state_sum"], rtol=1e-10)
    np.testing.assert_allclose(np.abs(sf).sum(), ref["final_state_abs_sum"], rtol=1e-12)
    np.testing.assert_allclose(np.abs(o).sum(), ref["o_abs_sum"], rtol=1e-12)


def test_input_recipe_shapes_and_ranges():
    spec, cu, x = kda_inputs.workload(4, tensors=("g",), T=4096, H=2)
    lens = np.diff(cu)
    assert cu[0] == 0 and cu[-1] == 4096 and lens.min() >= 1 and len(lens) == 64
    g = x["g"]
    assert np.all(g < 0) and g.dtype == np.float32
    # bf16-representable: low 16 bits of the float32 pattern are zero
    assert np.all((g.view(np.uint32) & 0xFFFF) == 0)
