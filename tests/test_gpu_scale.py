"""A caller-supplied logit scale (dims.sm_scale > 0) through the C ABI on an MI355X: the
prefill at both block sizes and the KAP builder against the fp64 oracles run at the
same scale (CoSA Eq. (1): S = Q K^T times the scale; Eq. (8) for KAP)."""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import kap, maskref
from tests.parity_helpers import check_prefill, delta_for_skip_fraction, gpu_to_host, oracle_arrays
from tests.test_gpu_kap import check_kap

pytestmark = pytest.mark.gpu

SCALE = 0.061  # about 0.7 / sqrt(128)
SHARP = 8.0     # about 90 / sqrt(128): logits spread over tens of units, peaked softmax rows


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


@pytest.mark.parametrize("block", [64, 128])
def test_prefill_with_caller_scale(rt, block):
    import torch
    wl = inputs.small_workload(f"scale{block}", [64 * 14 + 33, 200], 8, 2, generator="structured", seed=71,
                               pool="shuffled")
    bt = inputs.generate(dataclasses.replace(wl, block_size=block))
    q, k, _, pt, B = oracle_arrays(bt)
    om, ml = maskref.build_order_mask(q, k, pt, bt.cu_seqlens, 2, 0.5, page_size=B)
    delta = delta_for_skip_fraction(bt, om, ml, 0.3, sm_scale=SCALE)
    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws, sm_scale=SCALE)
    torch.cuda.synchronize()
    stats = check_prefill(bt, om, ml, delta, gpu_to_host(outs), sm_scale=SCALE)
    log("caller scale", block, stats)
    assert stats["skipped"] > 0


def test_kap_with_caller_scale(rt):
    wl = inputs.small_workload("scale_kap", [64 * 20 + 9], 8, 2, generator="structured", seed=72, pool="shuffled")
    check_kap(rt, "kap caller scale", inputs.generate(wl), 16, kap.MODE_TOP_P, 0.9, sm_scale=SCALE)


@pytest.mark.parametrize("block", [64, 128])
def test_prefill_with_sharp_logits(rt, block):
    # A large scale makes most rows' softmax nearly one-hot and moves the running max by
    # many units from page to page: the kernel's lazily moved exponent base must rescale
    # O and l often, and the output must still match the fp64 oracle.
    import torch
    wl = inputs.small_workload(f"sharp{block}", [64 * 16 + 7, 64 * 5], 8, 2, generator="iid", seed=73,
                               pool="shuffled")
    bt = inputs.generate(dataclasses.replace(wl, block_size=block))
    q, k, _, pt, B = oracle_arrays(bt)
    om, ml = maskref.build_order_mask(q, k, pt, bt.cu_seqlens, 2, 0.6, page_size=B)
    for frac in (0.0, 0.3):
        delta = delta_for_skip_fraction(bt, om, ml, frac, sm_scale=SHARP) if frac > 0 else -1.0
        db = rt.upload(bt)
        omd, mld = rt.upload_mask(om, ml)
        ws = rt.workspace_for(db, om.shape[2])
        outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws, sm_scale=SHARP)
        torch.cuda.synchronize()
        stats = check_prefill(bt, om, ml, delta, gpu_to_host(outs), sm_scale=SHARP)
        log("sharp logits", block, frac, stats)
        if frac > 0:
            assert stats["skipped"] > 0
