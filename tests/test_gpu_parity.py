"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on an MI355X.

Small shapes are compared in full (several tiles, ragged tails, packed sequences,
shuffled page pools, every head-group layout); the five measured workloads run
at full size in the launch configuration the benchmark times: the output of sampled
(query block, KV head) units is compared with the oracle's, and every skip decision
of the run with the oracle's decision log stored for that workload.
"""
import math
import os
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import maskref
from oracle.osk import full_causal_mask
from tests.oracle_helpers import random_masks
from tests.parity_helpers import (check_full_decision_log, check_mask_against_reference, check_prefill,
                                  delta_for_skip_fraction, gpu_to_host, host_arrays)

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


def run_and_check(rt, name, batch, om, ml, delta, units=None):
    import torch
    log(name, "seq_lens", batch.workload.seq_lens, "heads", batch.q.shape[1], batch.k_pool.shape[1],
        "mask", om.shape, "delta", delta)
    db = rt.upload(batch)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0, "inter-wave waits aborted"
    gpu = gpu_to_host(outs)
    stats = check_prefill(batch, om, ml, delta, gpu, units)
    log(name, stats)
    return stats, gpu


def oracle_mask(batch, b1, flags=3):
    q, k, _ = host_arrays(batch)
    return maskref.build_order_mask(q, k, batch.page_table, batch.cu_seqlens, batch.k_pool.shape[1], b1,
                                    flags=flags)


# --------------------------------------------------------------------------- small shapes
def test_small_mha_random_masks_with_junk(rt):
    wl = inputs.small_workload("mha1000", [1000], 1, 1, generator="structured", seed=11)
    bt = inputs.generate(wl)
    rng = np.random.default_rng(5)
    om, ml = random_masks(rng, [1000], 1, 64, 22, full_fraction=1.0)
    run_and_check(rt, "mha1000/off", bt, om, ml, -1.0)
    d = delta_for_skip_fraction(bt, om, ml, 0.4)
    st, _ = run_and_check(rt, "mha1000/skip", bt, om, ml, d)
    assert st["skipped"] > 0


@pytest.mark.parametrize("hq,hkv", [(8, 2), (2, 1), (3, 1), (16, 2), (4, 4)])
def test_small_gqa_packed_paged(rt, hq, hkv):
    lens = [200, 64, 130, 1, 520]
    wl = inputs.small_workload(f"gqa{hq}x{hkv}", lens, hq, hkv, generator="structured", seed=3 + hq,
                               pool="shuffled")
    bt = inputs.generate(wl)
    om, ml = oracle_mask(bt, 0.5)
    run_and_check(rt, f"gqa{hq}x{hkv}/off", bt, om, ml, -1.0)
    d = delta_for_skip_fraction(bt, om, ml, 0.4)
    st, _ = run_and_check(rt, f"gqa{hq}x{hkv}/skip", bt, om, ml, d)
    assert st["skipped"] > 0


def test_many_short_sequences(rt):
    # 48 packed sequences of random lengths (empty, one token, ragged tails, several
    # blocks): each unit finds its sequence by a search over cu_qblocks, its causal
    # range, its threshold ln(Delta / L_s) and its page-table row from its own entry.
    rng = np.random.default_rng(23)
    lens = [int(x) for x in rng.integers(0, 64 * 7, size=48)]
    lens[3], lens[17], lens[30] = 0, 1, 64
    wl = inputs.small_workload("many48", lens, 8, 2, generator="structured", seed=29, pool="shuffled")
    bt = inputs.generate(wl)
    log("case many48: lens", lens)
    om, ml = oracle_mask(bt, 0.5)
    run_and_check(rt, "many48/off", bt, om, ml, -1.0)
    d = delta_for_skip_fraction(bt, om, ml, 0.4)
    st, _ = run_and_check(rt, "many48/skip", bt, om, ml, d)
    assert st["skipped"] > 0


def test_empty_rows_junk_rows_and_all_skipped(rt):
    lens = [130, 70]
    wl = inputs.small_workload("edge", lens, 4, 1, generator="iid", seed=21)
    bt = inputs.generate(wl)
    om, ml = oracle_mask(bt, 0.5)
    om = np.concatenate([om, np.full((om.shape[0], 1, 3), -1, np.int32)], axis=2)
    ml = ml.copy()
    ml[0, 0] = 0                         # empty row: zero output, LSE -inf
    om[2, 0, :4] = [-1, 7, 3, 99]        # only junk: -1, non-causal, out of range
    ml[2, 0] = 4
    om[1, 0, :5] = [1, 0, 1, 0, -1]      # repeats
    ml[1, 0] = 5
    st, gpu = run_and_check(rt, "edge/off", bt, om, ml, -1.0)
    assert (gpu["out"][0:64] == 0).all() and np.isneginf(gpu["lse"][0:64]).all()
    # Delta above every sequence length skips every page: zero output everywhere
    st, gpu = run_and_check(rt, "edge/all-skipped", bt, om, ml, 1000.0)
    assert (gpu["out"] == 0).all() and np.isneginf(gpu["lse"]).all()


def test_dense_mask_small(rt):
    lens = [449, 64]
    wl = inputs.small_workload("dense", lens, 8, 2, generator="structured", seed=8)
    bt = inputs.generate(wl)
    om, ml = full_causal_mask(bt.cu_seqlens, 2)
    run_and_check(rt, "dense/off", bt, om.astype(np.int32), ml.astype(np.int32), -1.0)


def test_repeat_calls_are_bitwise_deterministic(rt):
    import torch
    wl = inputs.small_workload("det", [1000], 8, 2, generator="structured", seed=4)
    bt = inputs.generate(wl)
    om, ml = oracle_mask(bt, 0.3)
    d = delta_for_skip_fraction(bt, om, ml, 0.4)
    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    a = gpu_to_host(rt.prefill(db, omd, mld, d, log=True))
    b = gpu_to_host(rt.prefill(db, omd, mld, d, log=True))
    torch.cuda.synchronize()
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_validator_counts(rt):
    wl = inputs.small_workload("val", [300, 100], 4, 2, generator="iid", seed=2)
    bt = inputs.generate(wl)
    om, ml = oracle_mask(bt, 0.5)
    om = np.concatenate([om, np.full((om.shape[0], 2, 4), -1, np.int32)], axis=2)
    ml = ml.copy()
    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    assert (rt.validate_mask(db, omd, mld) == 0).all()
    # plant: an out-of-range id, a non-causal id, a repeat, a -1 inside the row, a bad length
    om[3, 1, ml[3, 1]] = 99; ml[3, 1] += 1
    om[2, 0, ml[2, 0]] = 4; ml[2, 0] += 1
    om[4, 1, ml[4, 1]] = om[4, 1, 0]; ml[4, 1] += 1
    om[1, 0, ml[1, 0]] = -1; ml[1, 0] += 1
    ml[0, 1] = -3                        # a negative length (treated as empty)
    omd, mld = rt.upload_mask(om, ml)
    got = rt.validate_mask(db, omd, mld)
    log("validator", got)
    assert list(got) == [2, 1, 1, 1, 0]


# --------------------------------------------------------------------------- mask builder
@pytest.mark.parametrize("b1,flags", [(0.5, 3), (0.25, 1), (0.2, 2), (0.0, 3), (1.0, 0)])
def test_mask_builder_small(rt, b1, flags):
    import torch
    wl = inputs.small_workload("mb", [700, 65, 300], 8, 2, generator="structured", seed=9, pool="shuffled")
    bt = inputs.generate(wl)
    q, k, _ = host_arrays(bt)
    ref_om, ref_ml, ref_sc = maskref.build_order_mask(q, k, bt.page_table, bt.cu_seqlens, 2, b1, flags=flags,
                                                      return_scores=True)
    db = rt.upload(bt)
    om, ml, sc = rt.build_mask(db, b1, flags=flags, width=ref_om.shape[2], scores=True)
    torch.cuda.synchronize()
    om, ml, sc = om.cpu().numpy(), ml.cpu().numpy(), sc.cpu().numpy()
    fin = np.isfinite(ref_sc)
    assert np.array_equal(fin, np.isfinite(sc))
    scale = np.abs(ref_sc[fin]).max()
    assert np.abs(sc[fin] - ref_sc[fin]).max() <= 1e-5 * scale
    n = check_mask_against_reference(om, ml, ref_om, ref_ml, ref_sc)
    log("builder small", b1, flags, "rows differing at near-ties:", n)


# --------------------------------------------------------------------------- the measured workloads
_CACHE = {}


def workload_case(name):
    if name not in _CACHE:
        wl = inputs.WORKLOADS[name]
        log(name, "generating inputs")
        bt = inputs.generate(wl)
        log(name, "oracle mask")
        om, ml = oracle_mask(bt, wl.budget1)
        _CACHE.clear()
        _CACHE[name] = (bt, om, ml, inputs.skip_scale(name))
    return _CACHE[name]


def sample_units(bt, n_blocks, seed):
    rng = np.random.default_rng(seed)
    nqb = bt.total_qblocks
    picks = set(rng.choice(nqb, size=min(n_blocks, nqb), replace=False).tolist())
    for s in range(bt.num_seqs):        # first and last block of every sequence
        picks |= {int(bt.cu_qblocks[s]), int(bt.cu_qblocks[s + 1] - 1)}
    return [(qb, g) for qb in sorted(picks) for g in range(bt.k_pool.shape[1])]


def _builder_parity(rt, name, bt, ref_om, ref_ml):
    import torch
    q, k, _ = host_arrays(bt)
    wl = inputs.WORKLOADS[name]
    log(name, "builder")
    db = rt.upload(bt)
    om, ml, sc = rt.build_mask(db, wl.budget1, width=ref_om.shape[2], scores=True)
    torch.cuda.synchronize()
    om, ml = om.cpu().numpy(), ml.cpu().numpy()
    # fp64 reference scores of every causal (block, page) pair
    prox = maskref.pooled_proxies(q, k, bt.page_table, bt.cu_seqlens, bt.k_pool.shape[1])
    ref_sc = np.full((bt.total_qblocks, bt.k_pool.shape[1], bt.max_blocks), np.nan)
    for s, (qbar, kbar) in enumerate(prox):
        base = bt.cu_qblocks[s]
        for g in range(bt.k_pool.shape[1]):
            full = qbar[:, g, :] @ kbar[:, g, :].T
            n = full.shape[0]
            ref_sc[base:base + n, g, :n] = np.where(np.tril(np.ones((n, n), bool)), full, np.nan)
    n = check_mask_against_reference(om, ml, ref_om, ref_ml, ref_sc)
    log(name, "builder rows differing at near-ties:", n, "of", ml.size)
    assert n <= max(1, ml.size // 100)


def test_cfg1_full(rt):
    bt, om, ml, d = workload_case("cfg1_2k_mha")
    st, _ = run_and_check(rt, "cfg1", bt, om, ml, d)
    assert st["visited"] == 303
    _builder_parity(rt, "cfg1_2k_mha", bt, om, ml)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["cfg2_16k_gqa", "cfg3_32k_structured", "cfg4_128k_structured",
                                  "cfg5_paged_2seq"])
def test_workload_full_size(rt, name):
    """Full-size run in the benchmark's launch configuration: the output of sampled
    units against the oracle, and every skip decision of the run against the oracle's
    stored decision log."""
    bt, om, ml, d = workload_case(name)
    units = sample_units(bt, 12, seed=len(name))
    st, gpu = run_and_check(rt, name, bt, om, ml, d, units=units)
    assert st["visited"] > 0
    full = check_full_decision_log(name, om, ml, bt.q.shape[1], gpu["decisions"])
    log(name, "full decision log:", full)
    _builder_parity(rt, name, bt, om, ml)
