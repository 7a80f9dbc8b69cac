"""Physical KV pages smaller than the logical block (CoSA Appendix D.1, "CoSA settings":
the block size and the KV-cache page size are set independently, so one logical block
may span several physical pages), through the C ABI on an MI355X.

Paging is storage only, so with the same tokens re-paged at 16 or 32 tokens per
physical page every result must be bitwise the one the 64-token layout gives: the
prefill's output, LSE, decision and margin logs, and the mean-pooled and KAP masks.
One case is also checked against the fp64 oracle on the logical view of the pool, and
a block with one unusable physical page must behave as an invalid logical id.
"""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import maskref, paging
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


def run_prefill(rt, batch, om, ml, delta):
    import torch
    db = rt.upload(batch)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    return gpu_to_host(outs)


def assert_same(a, b, what):
    for key in a:
        x, y = np.asarray(a[key]), np.asarray(b[key])
        assert x.shape == y.shape, (what, key)
        assert np.array_equal(x, y, equal_nan=True) if x.dtype.kind == "f" else np.array_equal(x, y), (what, key)


def logical_batch(bt, bp):
    kl, vl, ptl = paging.logical_view(bt.k_pool, bt.v_pool, bt.page_table, bt.cu_seqlens, bp)
    return dataclasses.replace(bt, k_pool=kl, v_pool=vl, page_table=ptl)


@pytest.mark.parametrize("bp", [16, 32])
def test_repaged_prefill_and_builders_are_bitwise_the_same(rt, bp):
    import torch
    wl = inputs.small_workload(f"pg{bp}", [64 * 21 + 37, 64 * 9, 30], 8, 2, generator="structured", seed=41,
                               pool="shuffled")
    bt64 = inputs.generate(wl)
    btp = inputs.repage(bt64, bp, 5)
    log("case", wl.name, "seq_lens", wl.seq_lens, "page", bp, "phys pages", btp.k_pool.shape[0])
    q, k, _ = host_arrays(bt64)
    om, ml = maskref.build_order_mask(q, k, bt64.page_table, bt64.cu_seqlens, 2, 0.5)
    delta = delta_for_skip_fraction(bt64, om, ml, 0.4)
    ref = run_prefill(rt, bt64, om, ml, delta)
    got = run_prefill(rt, btp, om, ml, delta)
    assert_same(ref, got, "prefill")
    stats = check_prefill(logical_batch(btp, bp), om, ml, delta, got)
    log("oracle on the logical view", stats)
    # the builders read keys through the physical pages too
    db64, dbp = rt.upload(bt64), rt.upload(btp)
    a = [x.cpu().numpy() for x in rt.build_mask(db64, 0.3, scores=True)]
    b = [x.cpu().numpy() for x in rt.build_mask(dbp, 0.3, scores=True)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    a = [x.cpu().numpy() for x in rt.build_kap_mask(db64, 16, 1, 0.9, outputs=True)]
    b = [x.cpu().numpy() for x in rt.build_kap_mask(dbp, 16, 1, 0.9, outputs=True)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    assert np.array_equal(rt.validate_mask(db64, *rt.upload_mask(om, ml)), rt.validate_mask(dbp, *rt.upload_mask(om, ml)))
    torch.cuda.synchronize()


def test_unusable_physical_page_invalidates_its_block(rt):
    wl = inputs.small_workload("pgbad", [64 * 12 + 9], 4, 1, generator="structured", seed=8, pool="identity")
    bt64 = inputs.generate(wl)
    btp = inputs.repage(bt64, 16, 3)
    bad = btp.page_table.copy()
    bad[0, 5 * 4 + 2] = -1                  # one of logical block 5's four physical pages
    btp_bad = dataclasses.replace(btp, page_table=bad)
    pt64_bad = bt64.page_table.copy()
    pt64_bad[0, 5] = -1
    bt64_bad = dataclasses.replace(bt64, page_table=pt64_bad)
    q, k, _ = host_arrays(bt64)
    om, ml = maskref.build_order_mask(q, k, bt64.page_table, bt64.cu_seqlens, 1, 0.6)
    delta = delta_for_skip_fraction(bt64, om, ml, 0.3)
    a = run_prefill(rt, bt64_bad, om, ml, delta)
    b = run_prefill(rt, btp_bad, om, ml, delta)
    assert_same(a, b, "invalid sub-page")
    # block 5 is never visited
    k_rows = np.argwhere(om[:, 0, :] == 5)
    assert k_rows.size and np.all(b["decisions"][k_rows[:, 0], :, k_rows[:, 1]] == 2)
    c64 = rt.validate_mask(rt.upload(bt64_bad), *rt.upload_mask(om, ml))
    cp = rt.validate_mask(rt.upload(btp_bad), *rt.upload_mask(om, ml))
    assert np.array_equal(c64, cp) and cp[4] > 0
    log("unusable sub-page: block 5 not visited in", k_rows.shape[0], "rows; validator", cp.tolist())


def test_full_size_128k_in_16_token_pages(rt):
    import torch
    wl64 = inputs.WORKLOADS["cfg4_128k_structured"]
    wl16 = inputs.WORKLOADS["cfg4_128k_structured_p16"]
    bt64, bt16 = inputs.generate(wl64), inputs.generate(wl16)
    db64, db16 = rt.upload(bt64), rt.upload(bt16)
    om, ml = rt.build_mask(db64, wl64.budget1)
    om16, ml16 = rt.build_mask(db16, wl16.budget1)
    assert torch.equal(om, om16) and torch.equal(ml, ml16)
    delta = inputs.skip_scale("cfg4_128k_structured")
    outs = []
    for db in (db64, db16):
        ws = rt.workspace_for(db, om.shape[2])
        o = rt.prefill(db, om, ml, delta, log=True, workspace=ws)
        torch.cuda.synchronize()
        assert rt.abort_count(db, ws, om.shape[2]) == 0
        outs.append(o)
    for name in ("out", "lse", "decisions", "margins"):
        x, y = getattr(outs[0], name), getattr(outs[1], name)
        same = torch.equal(torch.nan_to_num(x.float(), nan=-9.0), torch.nan_to_num(y.float(), nan=-9.0))
        assert same, name
    log("cfg4 128K in 16-token pages: bitwise equal to 64-token pages")


@pytest.mark.parametrize("block", [64, 128])
def test_pool_larger_than_a_phase(rt, block):
    # The launcher takes the KV heads in phases whose K and V pool slices fit 192 MiB (a
    # scheduling choice: it orders the units, nothing else).  A pool of 6,200 physical
    # pages gives 203 MB per KV head, so the two KV heads here run one after the other;
    # every result must be bitwise the one of the same tokens in a pool of their own
    # pages (one phase), and match the fp64 oracle.
    from tests.parity_helpers import oracle_arrays
    wl = inputs.small_workload(f"phases{block}", [64 * 23 + 11, 64 * 8], 8, 2, generator="structured", seed=43,
                               pool="shuffled")
    small = inputs.generate(dataclasses.replace(wl, block_size=block))
    big = inputs.generate(dataclasses.replace(wl, block_size=block, pool_pages=6200))
    per_head = big.k_pool.shape[0] * big.k_pool.shape[2] * big.k_pool.shape[3] * 2 * 2
    assert per_head > 192 << 20 > small.k_pool.shape[0] * 2 * per_head // big.k_pool.shape[0]
    log("case", wl.name, "block", block, "phys pages", small.k_pool.shape[0], "vs", big.k_pool.shape[0])
    q, k, _, pt, B = oracle_arrays(small)
    om, ml = maskref.build_order_mask(q, k, pt, small.cu_seqlens, 2, 0.5, page_size=B)
    delta = delta_for_skip_fraction(small, om, ml, 0.4)
    a = run_prefill(rt, small, om, ml, delta)
    b = run_prefill(rt, big, om, ml, delta)
    assert_same(a, b, "phases")
    stats = check_prefill(small, om, ml, delta, a)
    log("one phase vs two: bitwise equal; oracle", stats)
    assert stats["skipped"] > 0
