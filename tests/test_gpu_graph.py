"""The whole hot path -- the mean-pooled order-mask builder, the KAP builder and the
ordered-skipping prefill over the built mask -- captured once in a HIP graph (through
torch.cuda.CUDAGraph, on its capture stream) and replayed, on an MI355X.

Every launch of the library goes to the caller's stream, takes its scratch memory from
the caller's workspace, clears what must start at zero with kernels (no memset nodes),
and allocates nothing, so the calls can be captured.  Each replay, with eager work and
synchronisations in between, must give bitwise the eager results.
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


def test_builders_and_prefill_replay_in_a_graph(rt):
    import torch
    from block_sparse_long_osk_amd import binding
    wl = inputs.small_workload("graph", [64 * 40 + 7, 64 * 12, 33], 8, 2, generator="structured", seed=23,
                               pool="shuffled")
    db = rt.upload(inputs.generate(wl))
    budget = 0.3
    delta = 0.9 * float(64 * 40 + 7)  # threshold ln(Delta / L) about -0.1 on the longest sequence: skips happen
    width = binding.cosa_order_mask_width(db.max_blocks, budget)
    kw = binding.cosa_kap_mask_width(db.max_blocks, binding.COSA_KAP_TOP_P, 0.9)
    ws_b = torch.empty(binding.cosa_build_order_mask_workspace_bytes(db.dims(width)), dtype=torch.uint8, device="cuda")
    ws_k = torch.empty(binding.cosa_build_kap_mask_workspace_bytes(db.dims(kw)), dtype=torch.uint8, device="cuda")
    ws_p = rt.workspace_for(db, width)

    def path():
        om, ml = rt.build_mask(db, budget, width=width, workspace=ws_b)
        kom, kml = rt.build_kap_mask(db, 16, binding.COSA_KAP_TOP_P, 0.9, width=kw, workspace=ws_k)
        outs = rt.prefill(db, om, ml, delta, log=True, workspace=ws_p)
        return [om, ml, kom, kml, outs.out, outs.lse, outs.decisions, outs.margins]

    eager = [t.clone() for t in path()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = path()
    torch.cuda.synchronize()
    names = ["order_mask", "mask_len", "kap_order_mask", "kap_mask_len", "out", "lse", "decisions", "margins"]
    for rep in range(3):
        for t in captured:  # overwrite the graph's outputs so a stale replay cannot pass
            t.zero_()
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()  # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, eager, captured):
            if a.dtype.is_floating_point:
                same = torch.equal(torch.nan_to_num(a.float(), nan=-7.0), torch.nan_to_num(b.float(), nan=-7.0))
            else:
                same = torch.equal(a, b)
            assert same, (rep, name)
        log("replay", rep, "bitwise equal to the eager call")
    skipped = int((eager[6] == 1).sum().item())
    log("visits skipped in the captured prefill:", skipped)
    assert skipped > 0
