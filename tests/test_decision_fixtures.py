"""The stored full-size decision logs (oracle/decision_fixture.py) against the skip-scale
records (oracle/calibrate_skip_scale.py): both come from the fp64 oracle's margins of the
same seeded workloads, so the visit counts, skip ratios and near-tie counts must agree,
and each fixture's thresholds must be ln(Delta / L_s) of its workload (CoSA section 3.3,
Eq. (5))."""
import json
import math
import os

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import decision_fixture

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", decision_fixture.WORKLOADS)
def test_fixture_matches_its_workload(name):
    fx = decision_fixture.load(name)
    wl = inputs.WORKLOADS[name]
    assert fx["delta"] == inputs.skip_scale(name)
    assert np.allclose(fx["taus"], [math.log(fx["delta"] / L) for L in wl.seq_lens], rtol=0, atol=1e-12)
    assert fx["block"] == wl.block_size
    # one entry per visit: the row lengths of the mask at the workload's budget
    assert int(fx["mask_len"].sum()) * (wl.num_q_heads // wl.num_kv_heads) == fx["n"]
    assert fx["skip"].size == fx["near"].size == fx["n"]
    with open(os.path.join(ROOT, "block_sparse_long_osk_amd", "skip_scales.json")) as f:
        table = json.load(f)
    rec = table.get(name)
    if rec is not None:   # workloads calibrated at their own block size
        assert fx["n"] == rec["visits_per_q_head"]
        assert fx["skip"].mean() == pytest.approx(rec["skip_ratio"], abs=1e-12)
        assert int(fx["near"].sum()) == rec["near_tie_visits"]
