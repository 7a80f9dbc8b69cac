"""The longest-first schedule that cosa_osk_prefill builds before its attention kernel,
read back from the workspace (its first total_qblocks int32 words) on an MI355X.

Query blocks are visited in order of their mask length -- the largest over the KV heads,
clamped to [0, max_mask_len] -- longest first, equal lengths in ascending index order.
The schedule only orders work (any permutation gives the same attention output), so the
parity tests cannot see it; here it is compared exactly with a stable sort on the host,
for rows with few distinct lengths (many ties, one length bin per wave of the schedule
kernel) and with lengths spread over a few hundred bins.
"""
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs

pytestmark = pytest.mark.gpu


def log(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rt():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_long_osk_amd import binding, runner
    binding.lib()  # raises if the HIP library is missing: no fallback path exists
    return runner


def causal_rows(rng, nqb, hkv, width, lengths):
    """Mask rows of the given lengths: distinct causal blocks, the diagonal first."""
    om = np.full((nqb, hkv, width), -1, dtype=np.int32)
    ml = np.zeros((nqb, hkv), dtype=np.int32)
    for i in range(nqb):
        for g in range(hkv):
            n = min(int(lengths[i, g]), i + 1)
            rest = rng.choice(i, size=n - 1, replace=False) if n > 1 else np.zeros(0, dtype=np.int64)
            row = np.concatenate([[i], rest]).astype(np.int32) if n > 0 else np.zeros(0, dtype=np.int32)
            om[i, g, :n] = row
            ml[i, g] = n
    return om, ml


@pytest.mark.parametrize("name,width,choices", [("ties", 8, [0, 1, 2, 3, 5, 8]), ("spread", 300, None)])
def test_schedule_is_the_stable_longest_first_order(rt, name, width, choices):
    import torch
    nqb, hkv = 1500, 2
    log("case", name, "query blocks", nqb, "width", width)
    wl = inputs.small_workload(f"sched_{name}", [64 * nqb], 2, hkv, generator="iid", seed=5, pool="identity")
    batch = inputs.generate(wl)
    rng = np.random.default_rng(17)
    if choices is not None:
        lengths = rng.choice(choices, size=(nqb, hkv))
    else:
        lengths = rng.integers(0, width + 1, size=(nqb, hkv))
    om, ml = causal_rows(rng, nqb, hkv, width, lengths)
    db = rt.upload(batch)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, width)
    rt.prefill(db, omd, mld, 0.0, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, width) == 0
    got = ws[: 4 * nqb].cpu().numpy().view(np.int32)
    cost = np.clip(ml, 0, width).max(axis=1)
    want = np.argsort(-cost, kind="stable").astype(np.int32)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]
    log(name, "distinct lengths", len(np.unique(cost)), "schedule matches")
