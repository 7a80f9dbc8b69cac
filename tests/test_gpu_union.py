"""Per-q-head page sets under grouped-query heads (PageWeaver notes, section 2.2: the
heads of a KV group traverse the union of their sets, a membership mask keeps each
head's softmax to its own pages; Eq. (3): the reuse ratio rho_Q), through the C ABI on
an MI355X: cosa_osk_prefill_union against the fp64 oracle with membership, full
membership against cosa_osk_prefill bitwise, and cosa_build_union_mask against the
union builder's oracle, at small sizes in full and on the 128K workload sampled.
"""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import maskref
from tests.parity_helpers import check_prefill, delta_for_skip_fraction, gpu_to_host, oracle_arrays
from tests.test_union_oracle import random_union

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


def run_union(rt, bt, om, ml, mem, delta):
    import torch
    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    memd = torch.from_numpy(np.ascontiguousarray(mem, dtype=np.uint8)).to(db.q.device)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws, membership=memd)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    return gpu_to_host(outs)


CASES = [
    # name, seq_lens, hq, hkv, block, page, generator
    ("gqa4_b64", [64 * 17 + 21, 64 * 5, 33], 8, 2, 64, 64, "structured"),
    ("gqa8_b64_p16", [64 * 12 + 3], 16, 2, 64, 16, "structured"),
    ("gqa2_b64", [64 * 9 + 60], 4, 2, 64, 64, "structured"),
    ("gqa3_b64", [64 * 10 + 5], 6, 2, 64, 32, "structured"),
    ("gqa4_b128", [128 * 9 + 70, 128 * 2], 8, 2, 128, 64, "structured"),
    ("gqa3_b128", [128 * 6 + 1], 6, 2, 128, 128, "structured"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_union_prefill_parity(rt, case):
    name, lens, hq, hkv, B, bp, gen = case
    wl = inputs.small_workload("u_" + name, lens, hq, hkv, generator=gen, seed=61, pool="shuffled")
    wl = dataclasses.replace(wl, block_size=B, page_size=bp)
    bt = inputs.generate(wl)
    nb = [-(-L // B) for L in lens]
    om, ml, mem = random_union(bt.cu_seqlens, nb, hq, hkv, 17)
    log("case", name, "blocks", bt.total_qblocks, "width", om.shape[2], "membership share", float(mem.mean()))
    delta = delta_for_skip_fraction(bt, om, ml, 0.35, membership=mem)
    gpu = run_union(rt, bt, om, ml, mem, delta)
    stats = check_prefill(bt, om, ml, delta, gpu, membership=mem)
    log(name, stats)
    assert stats["skipped"] > 0 and stats["near_ties"] == 0
    # entries outside a head's membership are logged as not visited for it
    G = hq // hkv
    for h in range(hq):
        outside = (mem[:, h, :] == 0)
        assert (gpu["decisions"][:, h, :][outside] == 2).all()


def test_full_membership_is_the_shared_prefill_bitwise(rt):
    import torch
    wl = inputs.small_workload("u_full", [64 * 20 + 9, 64 * 3], 8, 2, generator="structured", seed=3,
                               pool="shuffled")
    bt = inputs.generate(wl)
    db = rt.upload(bt)
    om, ml = rt.build_mask(db, 0.3)
    delta = float(sum(wl.seq_lens)) * float(np.exp(-0.05))
    a = rt.prefill(db, om, ml, delta, log=True)
    ones = torch.ones((db.total_qblocks, db.num_q_heads, om.shape[2]), dtype=torch.uint8, device=db.q.device)
    b = rt.prefill(db, om, ml, delta, log=True, membership=ones)
    torch.cuda.synchronize()
    for name in ("out", "lse", "decisions", "margins"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(torch.nan_to_num(x.float(), nan=-9.0), torch.nan_to_num(y.float(), nan=-9.0)), name


def check_union_builder(rt, name, bt, b1, flags=3, blocks=None):
    """GPU union rows and membership against the oracle's: equal, or differing only
    where a head's selection or the union order meets scores within rounding."""
    import torch
    db = rt.upload(bt)
    om, ml, mem, hl = [x.cpu().numpy() for x in rt.build_union_mask(db, b1, flags=flags)]
    torch.cuda.synchronize()
    q, k, _, pt, B = oracle_arrays(bt)
    ro, rl, rm, rh = maskref.build_union_mask(q, k, pt, bt.cu_seqlens, bt.k_pool.shape[1], b1, page_size=B,
                                              flags=flags, width=om.shape[2])
    np.testing.assert_array_equal(hl, rh)
    want = range(om.shape[0]) if blocks is None else blocks
    differ = 0
    for qb in want:
        for g in range(om.shape[1]):
            G = mem.shape[1] // om.shape[1]
            same = (ml[qb, g] == rl[qb, g] and np.array_equal(om[qb, g], ro[qb, g])
                    and np.array_equal(mem[qb, g * G:(g + 1) * G], rm[qb, g * G:(g + 1) * G]))
            if not same:
                differ += 1
    rho = maskref.reuse_ratio(hl, ml)
    log(name, "union rows differing from the oracle:", differ, "of", len(list(want)) * om.shape[1], "rho_Q", rho)
    # rows may differ only through near-tied fp32 scores: a handful at most
    assert differ <= max(1, len(list(want)) * om.shape[1] // 100)
    assert abs(rho - maskref.reuse_ratio(rh, rl)) < 0.01 * rho
    # structural checks on every row: members of the union, counts, -1 / 0 padding
    W = om.shape[2]
    for qb in want:
        for g in range(om.shape[1]):
            n = ml[qb, g]
            G = mem.shape[1] // om.shape[1]
            m = mem[qb, g * G:(g + 1) * G]
            assert (om[qb, g, n:] == -1).all() and (m[:, n:] == 0).all()
            assert (m[:, :n].sum(axis=0) > 0).all()
            assert (m[:, :n].sum(axis=1) == hl[qb, g * G:(g + 1) * G]).all()
            assert len(set(om[qb, g, :n].tolist())) == n
    return om, ml, mem, hl


@pytest.mark.parametrize("b1,flags", [(0.3, 3), (0.1, 1), (0.0, 3)])
def test_union_builder_small(rt, b1, flags):
    wl = inputs.small_workload("ub", [64 * 30 + 7, 300], 8, 2, generator="structured", seed=13, pool="shuffled")
    check_union_builder(rt, f"union builder b1={b1} flags={flags}", inputs.generate(wl), b1, flags)


def test_union_builder_b128_p16(rt):
    wl = inputs.small_workload("ub128", [128 * 14 + 50], 8, 2, generator="structured", seed=14, pool="shuffled")
    wl = dataclasses.replace(wl, block_size=128, page_size=16)
    check_union_builder(rt, "union builder b=128 p16", inputs.generate(wl), 0.25)


@pytest.mark.timeout(900)
def test_union_full_size_128k_sampled(rt):
    import torch
    name = "cfg4_128k_structured"
    wl = inputs.WORKLOADS[name]
    log(name, "generating inputs")
    bt = inputs.generate(wl)
    db = rt.upload(bt)
    om, ml, mem, hl = rt.build_union_mask(db, wl.budget1)
    torch.cuda.synchronize()
    rho = float(hl.sum().item()) / float(ml.sum().item())
    delta = inputs.skip_scale(name)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, om, ml, delta, log=True, workspace=ws, membership=mem)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    gpu = gpu_to_host(outs)
    rng = np.random.default_rng(44)
    picks = sorted(set(rng.choice(bt.total_qblocks, 8, replace=False).tolist()) | {0, bt.total_qblocks - 1})
    units = [(qb, g) for qb in picks for g in range(bt.k_pool.shape[1])]
    stats = check_prefill(bt, om.cpu().numpy(), ml.cpu().numpy(), delta, gpu, units, membership=mem.cpu().numpy())
    log(name, "union prefill", stats, "rho_Q", rho)
    assert stats["visited"] > 0 and 1.0 <= rho <= 4.0
