"""The prefill at the largest inputs the library accepts, through the C ABI on an MI355X.

* 16,384 query blocks (the schedule kernel's and the no-allocation scratch's limit): 1,024
  packed sequences of 961..1,024 tokens (16 query blocks each, ragged tails) with two q
  heads on one KV head, a shuffled page pool and random ordered masks with junk entries.
* 16,384 logical blocks in one sequence (the limit of the visited-page bitmap): one
  sequence of 1,048,576 - 37 tokens, one head, rows of ids drawn over the whole causal
  range (repeats included, so the first-occurrence rule is exercised in every word of
  the bitmap).

Skipping on in both.  Checked: the longest-first schedule (read back from the workspace)
against a stable sort on the host; cosa_osk_prefill_noalloc bitwise against
cosa_osk_prefill on every output; and sampled (query block, KV head) units against the
fp64 oracle (output, LSE, decisions and margins), with the skip scale chosen from the
oracle's margins on those units.
"""
import math
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle.osk import osk_reference
from tests.oracle_helpers import random_masks
from tests.parity_helpers import check_prefill, gpu_to_host, oracle_arrays

pytestmark = pytest.mark.gpu

NUM_SEQS, WIDTH = 1024, 12


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


def delta_from_units(batch, om, ml, units, fraction=0.4):
    """A skip scale with about `fraction` of the sampled units' visits skipped, taken in a
    gap of at least 2e-3 between consecutive margins where there is one (so no sampled
    margin is a near-tie), from the oracle's decision-independent margins."""
    q, k, v, pt, B = oracle_arrays(batch)
    ref = osk_reference(q, k, v, pt, batch.cu_seqlens, om, ml, -1.0, page_size=B, compute_output=False,
                        units=units)
    lnL = np.zeros(om.shape[0])
    for s in range(len(batch.cu_seqlens) - 1):
        lnL[batch.cu_qblocks[s]:batch.cu_qblocks[s + 1]] = math.log(int(batch.cu_seqlens[s + 1] -
                                                                        batch.cu_seqlens[s]))
    m = ref["margins"]
    x = np.sort((m + lnL[:, None, None])[np.isfinite(m)])
    kq = int(round(fraction * x.size))
    splits = np.flatnonzero(np.diff(x) > 2e-3) + 1
    if splits.size:
        kq = int(splits[np.argmin(np.abs(splits - fraction * x.size))])
    return float(math.exp(0.5 * (x[kq - 1] + x[kq])))


def spread_rows(rng, n_blocks, width):
    """One sequence's rows: the diagonal block first, then width - 1 ids drawn uniformly
    (with repeats) from the causal blocks 0 .. i."""
    om = np.full((n_blocks, 1, width), -1, dtype=np.int64)
    ml = np.zeros((n_blocks, 1), dtype=np.int64)
    for i in range(n_blocks):
        om[i, 0, 0] = i
        om[i, 0, 1:] = rng.integers(0, i + 1, size=width - 1)
        ml[i, 0] = width
    return om, ml


def _case(name, rng):
    if name == "qblocks":
        lens = rng.integers(961, 1025, size=NUM_SEQS)
        wl = inputs.small_workload("limits", lens.tolist(), 2, 1, generator="iid", seed=91, pool="shuffled")
        bt = inputs.generate(wl)
        om, ml = random_masks(rng, lens.tolist(), 1, 64, WIDTH, junk=True, full_fraction=0.6)
        extra = {0, 1, 15, 16, bt.total_qblocks - 16, bt.total_qblocks - 1}
    else:
        wl = inputs.small_workload("limits_seq", [16384 * 64 - 37], 1, 1, generator="structured", seed=93,
                                   pool="shuffled")
        bt = inputs.generate(wl)
        om, ml = spread_rows(rng, bt.total_qblocks, WIDTH)
        extra = {0, 1, 2, 8191, 8192, 16382, 16383}
    picks = sorted(set(rng.choice(bt.total_qblocks, size=40, replace=False).tolist()) | extra)
    return bt, om, ml, [(qb, 0) for qb in picks]


@pytest.mark.parametrize("name", ["qblocks", "blocks_per_sequence"])
def test_largest_inputs_schedule_noalloc_and_oracle(rt, name):
    import torch
    from block_sparse_long_osk_amd import binding
    rng = np.random.default_rng(3)
    bt, om, ml, units = _case(name, rng)
    assert bt.total_qblocks == 16384
    delta = delta_from_units(bt, om, ml, units)
    log(name, "query blocks", bt.total_qblocks, "sequences", bt.num_seqs, "tokens", int(bt.cu_seqlens[-1]),
        "width", WIDTH, "delta", delta, "sampled units", len(units))

    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, WIDTH)
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, WIDTH) == 0
    ref = gpu_to_host(outs)

    # the schedule: longest first by the largest clamped mask length over the KV heads, stable
    got = ws[: 4 * bt.total_qblocks].cpu().numpy().view(np.int32)
    want = np.argsort(-np.clip(ml, 0, WIDTH).max(axis=1), kind="stable").astype(np.int32)
    assert np.array_equal(got, want)
    log("schedule of 16384 query blocks equals the stable host sort")

    # the entry point that allocates nothing, at the largest input its scratch holds
    assert binding.cosa_osk_workspace_bytes(db.dims(WIDTH)) <= binding.COSA_OSK_NOALLOC_SCRATCH_BYTES
    na = rt.allocate_outputs(db, WIDTH, log=True)
    binding.cosa_osk_prefill_noalloc(db.dims(WIDTH), db.q, db.k_pool, db.v_pool, db.page_table, db.cu_seqlens,
                                     db.cu_qblocks, omd, mld, delta, na.out, na.lse, na.decisions, na.margins)
    torch.cuda.synchronize()
    got_na = gpu_to_host(na)
    for key in ("out", "lse", "decisions", "margins"):
        assert np.array_equal(got_na[key], ref[key], equal_nan=True), key
    log("cosa_osk_prefill_noalloc bitwise equal at 16384 query blocks")

    dec = ref["decisions"]
    assert (dec == 1).any() and (dec == 0).any()
    stats = check_prefill(bt, om, ml, delta, ref, units=units)
    log("against the oracle:", stats)
