"""Page-table entries that name no page of the physical pool, HIP path against the fp64
oracle, through the C ABI on an MI355X.

PageWeaver notes, section 2.1 (conventions): an id that does not name a stored page
adds no interaction.  A page-table entry of -1, or one at or past the pool size,
makes its logical block unusable: the prefill does not visit it (decision code 2) and
the builders see no stored keys there.  The mask rows come from the valid page table,
so they name the unusable blocks; the oracle and the kernels then receive the page
table with the bad entries, at 64-token blocks over 64- and 16-token pages and at
128-token blocks over 64-token pages.
"""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import kap, maskref
from tests.parity_helpers import (check_mask_against_reference, check_prefill, delta_for_skip_fraction,
                                  gpu_to_host, oracle_arrays)
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


# name, seq_lens, hq, hkv, block, page, bad entries: (sequence, page-table column, kind)
CASES = [
    ("b64_p64", [64 * 11 + 20, 64 * 6], 8, 2, 64, 64, [(0, 3, "neg"), (0, 9, "past"), (1, 2, "neg")]),
    ("b64_p16", [64 * 9 + 5, 64 * 4 + 50], 8, 2, 64, 16, [(0, 4 * 2 + 1, "neg"), (1, 4 * 3, "past")]),
    ("b128_p64", [128 * 7 + 40, 128 * 3], 8, 2, 128, 64, [(0, 2 * 2 + 1, "neg"), (0, 2 * 5, "past"),
                                                           (1, 2, "neg")]),
]


def make_case(case):
    name, lens, hq, hkv, block, page, bad = case
    wl = inputs.small_workload("unmapped_" + name, lens, hq, hkv, generator="structured", seed=61,
                               pool="shuffled")
    wl = dataclasses.replace(wl, block_size=block, page_size=page,
                             pool_seed=wl.pool_seed if wl.pool_seed is not None else 63)
    good = inputs.generate(wl)
    pt = good.page_table.copy()
    n_phys = good.k_pool.shape[0]
    for s, col, kind in bad:
        assert pt[s, col] >= 0
        pt[s, col] = -1 if kind == "neg" else n_phys + 2
    return good, dataclasses.replace(good, page_table=pt)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_skips_unmapped_blocks_like_the_oracle(rt, case):
    import torch
    good, bad = make_case(case)
    log("case", case[0], "seq_lens", good.workload.seq_lens, "bad entries", case[6])
    q, k, _, pt_good, B = oracle_arrays(good)
    om, ml = maskref.build_order_mask(q, k, pt_good, good.cu_seqlens, good.k_pool.shape[1], 0.5, page_size=B)
    # the blocks the oracle's view of the bad table cannot use (an entry outside its pool)
    _, k_bad, _, pt_bad_log, _ = oracle_arrays(bad)
    no_page = (pt_bad_log < 0) | (pt_bad_log >= k_bad.shape[0])
    unusable = sum(int(row[: -(-int(L) // B)].sum()) for row, L in zip(no_page, np.diff(bad.cu_seqlens)))
    assert unusable == len({(s, col * case[5] // B) for s, col, _ in case[6]})
    delta = delta_for_skip_fraction(bad, om, ml, 0.4)
    db = rt.upload(bad)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    gpu = gpu_to_host(outs)
    stats = check_prefill(bad, om, ml, delta, gpu)
    # every entry that names an unusable block is logged as not visited by every head
    G = good.q.shape[1] // good.k_pool.shape[1]
    cu_qb = bad.cu_qblocks
    n_bad_entries = 0
    for qb in range(om.shape[0]):
        s = int(np.searchsorted(cu_qb, qb, side="right") - 1)
        for g in range(om.shape[1]):
            for kk in range(int(ml[qb, g])):
                if no_page[s, om[qb, g, kk]]:
                    n_bad_entries += 1
                    assert np.all(gpu["decisions"][qb, g * G:(g + 1) * G, kk] == 2)
    assert n_bad_entries > 0
    assert stats["skipped"] > 0
    log(case[0], "entries naming unusable blocks:", n_bad_entries, stats)
    # the validator counts them
    counts = rt.validate_mask(db, omd, mld)
    assert counts[4] == n_bad_entries, counts


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_builders_see_no_keys_on_unmapped_blocks(rt, case):
    import torch
    _, bad = make_case(case)
    q, k, _, pt, B = oracle_arrays(bad)
    hkv = bad.k_pool.shape[1]
    ref_om, ref_ml, ref_sc = maskref.build_order_mask(q, k, pt, bad.cu_seqlens, hkv, 0.5, page_size=B,
                                                      return_scores=True)
    db = rt.upload(bad)
    om, ml, sc = rt.build_mask(db, 0.5, width=ref_om.shape[2], scores=True)
    torch.cuda.synchronize()
    om, ml, sc = om.cpu().numpy(), ml.cpu().numpy(), sc.cpu().numpy()
    fin = np.isfinite(ref_sc)
    assert np.array_equal(fin, np.isfinite(sc))
    scale = np.abs(ref_sc[fin]).max()
    assert np.abs(sc[fin] - ref_sc[fin]).max() <= 1e-5 * scale
    n = check_mask_against_reference(om, ml, ref_om, ref_ml, ref_sc)
    log(case[0], "mean-pooled builder rows differing at near-ties:", n)
    check_kap(rt, "unmapped_kap_" + case[0], bad, 16, kap.MODE_FRACTION, 0.4)
    check_kap(rt, "unmapped_kap_topp_" + case[0], bad, 16, kap.MODE_TOP_P, 0.9)
