"""The oracle reproduces its committed snapshot (regression anchor, see tests/golden/README.md)."""
import json
import os

import numpy as np
import pytest

import oracle
from dynamic_dilated_depthwise_amd import synth

SNAP = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_snapshot.json")


@pytest.mark.parametrize("name", ["tiny", "nonaligned"])
def test_oracle_matches_snapshot(name):
    doc = json.load(open(SNAP))["cases"][name]
    shape, block = synth.WORKLOADS[name]
    assert doc["shape"] == [shape.N, shape.C, shape.H, shape.W, shape.K]
    t = synth.make_inputs(shape, block, grad=True, taps=True)
    a = {k: v.double().numpy() for k, v in t.items()}
    orc = oracle.default()
    got = {"fused_fwd": orc.fused_fwd(a["x"], a["y"], a["weight"], a["bias"], shape.K),
           "filter_fwd": orc.filter_fwd(a["x"], a["taps"], shape.K)}
    got.update(zip(("dx", "dy", "dweight", "dbias"),
                   orc.fused_bwd(a["x"], a["y"], a["weight"], a["bias"], a["grad_out"], shape.K)))
    for key, arr in got.items():
        flat = arr.reshape(-1)
        ref = doc[key]
        np.testing.assert_allclose(flat[ref["index"]], ref["value"], rtol=1e-12, atol=1e-12, err_msg=key)
        np.testing.assert_allclose(flat.sum(), ref["sum"], rtol=1e-10, atol=1e-10, err_msg=key)
