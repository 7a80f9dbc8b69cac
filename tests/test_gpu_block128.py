"""128-token logical blocks (CoSA Appendix D.1: b = 128 for queries, keys and values
alike, one skip vote per 128-row query tile, each block found through the physical
pages of the paged KV cache), through the C ABI on an MI355X.

The prefill is checked against the fp64 oracle run at page size 128 on the logical
view of the pool, for physical pages of 16, 32, 64 and 128 tokens, ragged tails that
end inside either 64-token half of the last block, grouped and ungrouped heads, junk
mask entries, skipping on and off; the same tokens under the four page sizes must
give bitwise the same results.  The mean-pooled and KAP builders at b = 128 are held
to their oracles as at b = 64, and the 128K workload is run at full size with sampled
units checked.
"""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import kap, maskref, osk
from tests.parity_helpers import (check_full_decision_log, check_mask_against_reference, check_prefill,
                                  delta_for_skip_fraction, gpu_to_host, oracle_arrays)
from tests.test_gpu_kap import check_kap

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


def workload(name, lens, hq, hkv, page_size, gen="structured", pool="shuffled", seed=31, budget1=0.5):
    wl = inputs.small_workload(name, lens, hq, hkv, generator=gen, seed=seed, pool=pool, budget1=budget1)
    return dataclasses.replace(wl, block_size=128, page_size=page_size,
                               pool_seed=wl.pool_seed if wl.pool_seed is not None else seed + 2)


def oracle_mask(bt, b1, flags=3, scores=False):
    q, k, _, pt, B = oracle_arrays(bt)
    return maskref.build_order_mask(q, k, pt, bt.cu_seqlens, bt.k_pool.shape[1], b1, page_size=B, flags=flags,
                                    return_scores=scores)


def run_prefill(rt, bt, om, ml, delta):
    import torch
    db = rt.upload(bt)
    assert db.block_size == 128
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    return gpu_to_host(outs)


CASES = [
    # name, seq_lens, hq, hkv, page size, generator, pool
    ("gqa4_p64", [128 * 9 + 37, 128 * 3 + 64, 100], 8, 2, 64, "structured", "shuffled"),
    ("gqa4_p16", [128 * 6 + 70, 128 * 2], 8, 2, 16, "structured", "shuffled"),
    ("gqa4_p32", [128 * 5 + 1], 8, 2, 32, "iid", "identity"),
    ("gqa4_p128", [128 * 7 + 127, 64], 8, 2, 128, "structured", "shuffled"),
    ("mha_p64", [128 * 10 + 65], 2, 2, 64, "structured", "identity"),
    ("gqa3_p32", [128 * 3 + 10, 300], 6, 2, 32, "structured", "shuffled"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_b128_prefill_parity(rt, case):
    name, lens, hq, hkv, bp, gen, pool = case
    wl = workload("b128_" + name, lens, hq, hkv, bp, gen, pool)
    bt = inputs.generate(wl)
    log("case", name, "seq_lens", lens, "heads", hq, hkv, "page", bp, "blocks", bt.total_qblocks)
    om, ml = oracle_mask(bt, 0.5)
    # junk entries: a repeat, a -1, an id past the sequence's blocks, a non-causal id
    width = om.shape[2]
    om = np.concatenate([om, np.full((om.shape[0], hkv, 4), -1, np.int32)], axis=2)
    last = bt.total_qblocks - 1
    for qb, g, junk in ((last, 0, [int(om[last, 0, 0]), -1, 10 ** 6]), (0, hkv - 1, [1, 0])):
        n = int(ml[qb, g])
        om[qb, g, n:n + len(junk)] = junk
        ml[qb, g] = n + len(junk)
    assert om.shape[2] >= width
    delta = delta_for_skip_fraction(bt, om, ml, 0.4)
    gpu = run_prefill(rt, bt, om, ml, delta)
    stats = check_prefill(bt, om, ml, delta, gpu)
    log(name, stats)
    assert stats["skipped"] > 0
    # skipping off on the dense causal mask
    omd, mld = osk.full_causal_mask(bt.cu_seqlens, hkv, page_size=128)
    gpu = run_prefill(rt, bt, omd, mld, -1.0)
    stats = check_prefill(bt, omd, mld, -1.0, gpu)
    log(name, "dense", stats)
    assert stats["skipped"] == 0


def test_b128_page_size_is_storage_only(rt):
    wl64 = workload("b128_pages", [128 * 11 + 90, 128 * 2 + 5], 8, 2, 64)
    bt64 = inputs.generate(wl64)
    om, ml = oracle_mask(bt64, 0.4)
    delta = delta_for_skip_fraction(bt64, om, ml, 0.4)
    ref = run_prefill(rt, bt64, om, ml, delta)
    for bp in (16, 32, 128):
        btp = inputs.repage(bt64, bp, 7 + bp)
        got = run_prefill(rt, btp, om, ml, delta)
        for key in ref:
            assert np.array_equal(ref[key], got[key], equal_nan=True), (bp, key)
    log("b128: pages of 16, 32, 64, 128 tokens give bitwise the same prefill")


@pytest.mark.parametrize("bp", [64, 16])
def test_b128_mean_pooled_builder(rt, bp):
    import torch
    wl = workload(f"b128_mb{bp}", [128 * 13 + 20, 129, 60], 8, 2, bp)
    bt = inputs.generate(wl)
    for b1, flags in ((0.5, 3), (0.2, 1), (0.0, 3)):
        ref_om, ref_ml, ref_sc = oracle_mask(bt, b1, flags=flags, scores=True)
        db = rt.upload(bt)
        om, ml, sc = rt.build_mask(db, b1, flags=flags, width=ref_om.shape[2], scores=True)
        torch.cuda.synchronize()
        om, ml, sc = om.cpu().numpy(), ml.cpu().numpy(), sc.cpu().numpy()
        fin = np.isfinite(ref_sc)
        assert np.array_equal(fin, np.isfinite(sc))
        assert np.abs(sc[fin] - ref_sc[fin]).max() <= 1e-5 * np.abs(ref_sc[fin]).max()
        n = check_mask_against_reference(om, ml, ref_om, ref_ml, ref_sc)
        log("b128 builder", bp, b1, flags, "rows differing at near-ties:", n)
        # and the validator counts nothing wrong in it
        assert list(rt.validate_mask(db, *rt.upload_mask(om, ml))) == [0, 0, 0, 0, 0]


KAP_CASES = [
    # name, seq_lens, hq, hkv, page size, stride, mode, budget
    ("s16_frac", [128 * 18 + 13, 128 * 3], 8, 2, 64, 16, kap.MODE_FRACTION, 0.3),
    ("s32_topp", [128 * 18 + 13, 128 * 3], 8, 2, 16, 32, kap.MODE_TOP_P, 0.9),
    ("s16_mha", [128 * 10 + 100], 2, 2, 128, 16, kap.MODE_TOP_P, 0.8),
    ("s32_gqa8", [128 * 7 + 5], 16, 2, 32, 32, kap.MODE_FRACTION, 0.25),
]


@pytest.mark.parametrize("case", KAP_CASES, ids=[c[0] for c in KAP_CASES])
def test_b128_kap_builder(rt, case):
    name, lens, hq, hkv, bp, stride, mode, budget = case
    log("case", name, lens, hq, hkv, bp, stride, mode, budget)
    bt = inputs.generate(workload("b128_kap_" + name, lens, hq, hkv, bp, seed=77))
    check_kap(rt, "b128_" + name, bt, stride, mode, budget)


def test_b128_rejects_unsupported(rt):
    import torch
    from block_sparse_long_osk_amd import binding
    bt = inputs.generate(workload("b128_rej", [128 * 3], 8, 2, 64, seed=1))
    db = rt.upload(bt)
    with pytest.raises(binding.CosaError):
        rt.build_kap_mask(db, 8, kap.MODE_FRACTION, 0.5)   # 16 samples per block: not supported
    torch.cuda.synchronize()


@pytest.mark.timeout(900)
def test_b128_full_size_128k(rt):
    import torch
    name = "cfg4_128k_structured_b128"
    wl = inputs.WORKLOADS[name]
    log(name, "generating inputs")
    bt = inputs.generate(wl)
    log(name, "oracle mask")
    ref_om, ref_ml, ref_sc = oracle_mask(bt, wl.budget1, scores=True)
    db = rt.upload(bt)
    om, ml = rt.build_mask(db, wl.budget1, width=ref_om.shape[2])
    torch.cuda.synchronize()
    n = check_mask_against_reference(om.cpu().numpy(), ml.cpu().numpy(), ref_om, ref_ml, ref_sc)
    log(name, "builder rows differing at near-ties:", n, "of", ml.numel())
    assert n <= max(1, ml.numel() // 100)
    delta = inputs.skip_scale(name)
    gpu = run_prefill(rt, bt, ref_om, ref_ml, delta)
    rng = np.random.default_rng(128)
    picks = sorted(set(rng.choice(bt.total_qblocks, 10, replace=False).tolist()) | {0, bt.total_qblocks - 1})
    units = [(qb, g) for qb in picks for g in range(bt.k_pool.shape[1])]
    stats = check_prefill(bt, ref_om, ref_ml, delta, gpu, units)
    log(name, stats)
    assert stats["visited"] > 0
    full = check_full_decision_log(name, ref_om, ref_ml, bt.q.shape[1], gpu["decisions"])
    log(name, "full decision log:", full)
