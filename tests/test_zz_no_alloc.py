"""cosa_osk_prefill_noalloc (the prefill for callers that cannot allocate: its
workspace is a library-held device array) against cosa_osk_prefill, through the C
ABI on an MI355X.

Two calls in a row share the library's scratch, the second on a smaller input than
the first: each must give bitwise the output, LSE, decision log and margins of
cosa_osk_prefill with a caller-owned workspace on the same inputs (the kernels are
the same), and the first is also held to the fp64 oracle.
"""
import ctypes
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import maskref
from tests.parity_helpers import check_prefill, delta_for_skip_fraction, gpu_to_host, host_arrays

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


def _case(name, lens, hq, hkv, seed, b1):
    wl = inputs.small_workload(name, lens, hq, hkv, generator="structured", seed=seed, pool="shuffled")
    bt = inputs.generate(wl)
    q, k, _ = host_arrays(bt)
    om, ml = maskref.build_order_mask(q, k, bt.page_table, bt.cu_seqlens, hkv, b1)
    return bt, om, ml, delta_for_skip_fraction(bt, om, ml, 0.4)


def _noalloc(rt, db, omd, mld, delta, width):
    from block_sparse_long_osk_amd import binding
    outs = rt.allocate_outputs(db, width, log=True)
    binding.cosa_osk_prefill_noalloc(db.dims(width), db.q, db.k_pool, db.v_pool, db.page_table, db.cu_seqlens,
                                     db.cu_qblocks, omd, mld, delta, outs.out, outs.lse, outs.decisions,
                                     outs.margins)
    return outs


def test_noalloc_matches_workspace_entry_on_two_calls(rt):
    import torch
    big = _case("noalloc_big", [64 * 29 + 17, 300, 64 * 11], 8, 2, 71, 0.4)
    small = _case("noalloc_small", [64 * 5 + 3, 70], 8, 2, 72, 0.5)
    assert big[0].total_qblocks > small[0].total_qblocks
    for name, (bt, om, ml, delta) in (("big", big), ("small", small)):
        log("case", name, "seq_lens", bt.workload.seq_lens, "qblocks", bt.total_qblocks, "delta", delta)
        db = rt.upload(bt)
        omd, mld = rt.upload_mask(om, ml)
        width = om.shape[2]
        ref = gpu_to_host(rt.prefill(db, omd, mld, delta, log=True))
        got_dev = _noalloc(rt, db, omd, mld, delta, width)
        torch.cuda.synchronize()
        got = gpu_to_host(got_dev)
        for key in ("out", "lse", "decisions", "margins"):
            assert np.array_equal(got[key], ref[key], equal_nan=True), (name, key)
        assert (got["decisions"] == 1).any() and (got["decisions"] == 0).any()
        if name == "big":
            stats = check_prefill(bt, om, ml, delta, got)
            log(name, "against the oracle:", stats)
        log(name, "bitwise equal to cosa_osk_prefill")


def test_noalloc_rejects_shapes_beyond_its_scratch(rt):
    from block_sparse_long_osk_amd import binding
    bt = _case("noalloc_rej", [64 * 3], 4, 1, 73, 0.5)[0]
    db = rt.upload(bt)
    dims = db.dims(4)
    assert binding.cosa_osk_workspace_bytes(dims) <= binding.COSA_OSK_NOALLOC_SCRATCH_BYTES
    dims.total_qblocks = 16385                 # past the query blocks the scratch holds
    dims.total_q_tokens = 16385 * 64
    st = binding.lib().cosa_osk_prefill_noalloc(ctypes.byref(dims), *([None] * 8), ctypes.c_float(-1.0),
                                                *([None] * 5))
    assert st < 0
