"""Concurrent calls: the library keeps no state between or across calls (each call's
scratch is its caller's workspace), so prefill calls issued at once from two host threads,
each on its own stream with its own workspace and outputs, give bitwise the results of the
same calls made one after the other on one stream; on an MI355X.

Streams are created at the default priority.  The two batches differ in shape (packed
sequences, head layouts, page pools), so a call that read another's schedule, mask window
or outputs would not go unnoticed.
"""
import sys
import threading

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


def test_concurrent_calls_on_two_streams_match_sequential_calls(rt):
    import torch
    cases = [_case("streams_a", [64 * 40 + 9, 300, 64 * 7], 8, 2, 81, 0.4),
             _case("streams_b", [64 * 23, 64 * 31 + 50], 12, 4, 82, 0.5)]
    prepared = []
    for bt, om, ml, delta in cases:
        db = rt.upload(bt)
        omd, mld = rt.upload_mask(om, ml)
        prepared.append((bt, om, ml, delta, db, omd, mld))
    torch.cuda.synchronize()

    # one after the other, on the current stream
    ref = []
    for bt, om, ml, delta, db, omd, mld in prepared:
        ref.append(gpu_to_host(rt.prefill(db, omd, mld, delta, log=True)))
    torch.cuda.synchronize()

    # at once: each host thread issues REPEATS calls on its own stream
    REPEATS = 4
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = [[None] * REPEATS for _ in prepared]
    errors = []

    def worker(x):
        try:
            bt, om, ml, delta, db, omd, mld = prepared[x]
            with torch.cuda.stream(streams[x]):
                for r in range(REPEATS):
                    ws = rt.workspace_for(db, om.shape[2])
                    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws, stream=streams[x])
                    results[x][r] = (outs, ws)
            streams[x].synchronize()
        except Exception as e:  # reported from the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(x,)) for x in range(len(prepared))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a calling thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()

    for x, (bt, om, ml, delta, db, omd, mld) in enumerate(prepared):
        for r in range(REPEATS):
            outs, ws = results[x][r]
            assert rt.abort_count(db, ws, om.shape[2]) == 0
            got = gpu_to_host(outs)
            for key in ("out", "lse", "decisions", "margins"):
                assert np.array_equal(got[key], ref[x][key], equal_nan=True), (x, r, key)
        log(bt.workload.name, f"{REPEATS} concurrent calls bitwise equal to the sequential call")
        stats = check_prefill(bt, om, ml, delta, ref[x])
        log(bt.workload.name, "against the oracle:", stats)
