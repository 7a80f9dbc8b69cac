"""Edge shapes through the C ABI on an MI355X, against the fp64 oracle: an empty and a
one-token sequence packed between ragged ones; mask rows far longer than one resolve
window (512 entries, 256 or 128 when a block spans several physical pages), with
repeated ids whose first occurrence lies in an earlier window and valid first
occurrences only in late windows; and the widest row the library accepts (8191)."""
import dataclasses
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import maskref
from tests.parity_helpers import check_prefill, delta_for_skip_fraction, gpu_to_host, oracle_arrays

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


def run(rt, bt, om, ml, delta):
    import torch
    db = rt.upload(bt)
    omd, mld = rt.upload_mask(om, ml)
    ws = rt.workspace_for(db, om.shape[2])
    outs = rt.prefill(db, omd, mld, delta, log=True, workspace=ws)
    torch.cuda.synchronize()
    assert rt.abort_count(db, ws, om.shape[2]) == 0
    return gpu_to_host(outs)


def test_empty_and_one_token_sequences(rt):
    wl = inputs.small_workload("edge_len", [64 * 9 + 5, 0, 1, 64 * 3, 0, 65], 8, 2, generator="structured", seed=12,
                               pool="shuffled")
    bt = inputs.generate(wl)
    assert list(np.diff(bt.cu_qblocks)) == [10, 0, 1, 3, 0, 2]
    q, k, _, pt, B = oracle_arrays(bt)
    om, ml = maskref.build_order_mask(q, k, pt, bt.cu_seqlens, 2, 0.5)
    delta = delta_for_skip_fraction(bt, om, ml, 0.3)
    gpu = run(rt, bt, om, ml, delta)
    stats = check_prefill(bt, om, ml, delta, gpu)
    log("empty and one-token sequences", stats)


def long_rows(bt, width, seed):
    """Rows of `width` entries: junk and repeats first, then every causal block once in
    random order, then repeats again -- so the valid first occurrences fall in late
    windows and repeats straddle windows."""
    rng = np.random.default_rng(seed)
    hkv = bt.k_pool.shape[1]
    nqb = bt.total_qblocks
    om = np.full((nqb, hkv, width), -1, np.int32)
    ml = np.zeros((nqb, hkv), np.int32)
    B = bt.block_size
    for s in range(bt.num_seqs):
        L = int(bt.cu_seqlens[s + 1] - bt.cu_seqlens[s])
        n = -(-L // B)
        for i in range(n):
            qb = int(bt.cu_qblocks[s]) + i
            for g in range(hkv):
                ids = rng.permutation(i + 1)
                keep = ids[: max(1, (i + 1) // 2)]
                head = rng.choice([-1, n + 5, 10 ** 6], size=width // 2 - 3).astype(np.int64)
                if i > 0:
                    head[::7] = i + 1 if i + 1 < n else -2      # non-causal ids
                body = keep
                tail = rng.choice(keep, size=width - len(head) - len(body))  # repeats only
                row = np.concatenate([head, body, tail])[:width]
                om[qb, g, :] = row
                ml[qb, g] = width
    return om, ml


@pytest.mark.parametrize("block,page", [(64, 64), (64, 16), (128, 64), (128, 16)])
def test_rows_longer_than_many_windows(rt, block, page):
    wl = inputs.small_workload("edge_win", [64 * 12 + 17], 8, 2, generator="structured", seed=21, pool="shuffled")
    wl = dataclasses.replace(wl, block_size=block, page_size=page)
    bt = inputs.generate(wl)
    om, ml = long_rows(bt, 2100, 5)
    delta = delta_for_skip_fraction(bt, om, ml, 0.3)
    gpu = run(rt, bt, om, ml, delta)
    stats = check_prefill(bt, om, ml, delta, gpu)
    log("long rows", block, page, stats)
    assert stats["visited"] > 0


def test_widest_rows(rt):
    wl = inputs.small_workload("edge_wide", [64 * 5 + 3], 4, 1, generator="structured", seed=33, pool="identity")
    bt = inputs.generate(wl)
    om, ml = long_rows(bt, 8191, 9)
    delta = delta_for_skip_fraction(bt, om, ml, 0.3)
    gpu = run(rt, bt, om, ml, delta)
    stats = check_prefill(bt, om, ml, delta, gpu)
    log("widest rows", stats)


def test_empty_batch(rt):
    """Every sequence empty (no query blocks, a page table of no columns): the prefill and the
    mask builder launch nothing and return, with torch's empty tensors as arguments."""
    import torch
    from block_sparse_long_osk_amd import binding
    wl = inputs.small_workload("empty_batch", [0, 0, 0], 4, 1, generator="structured", seed=5, pool="shuffled")
    bt = inputs.generate(wl)
    assert bt.total_qblocks == 0
    log("empty batch: seq_lens", bt.workload.seq_lens, "page table", bt.page_table.shape)
    db = rt.upload(bt)
    om = np.zeros((0, 1, 4), dtype=np.int32)
    ml = np.zeros((0, 1), dtype=np.int32)
    omd, mld = rt.upload_mask(om, ml)
    outs = rt.prefill(db, omd, mld, 100.0, log=True)
    torch.cuda.synchronize()
    assert tuple(outs.out.shape) == (0, 4, 128) and tuple(outs.decisions.shape) == (0, 4, 4)
    bm, bl = rt.build_mask(db, 0.5, width=4)
    torch.cuda.synchronize()
    assert bm.shape[0] == 0 and bl.shape[0] == 0
    assert binding.cosa_abi_version() == 2
