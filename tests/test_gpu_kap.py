"""Parity of the KAP mask builder (cosa_build_kap_mask, through the C ABI) with the
fp64 KAP oracle (CoSA section 4.2, Eq. (8)-(14)), on an MI355X.

The kernel's block scores must match the oracle's to 1e-5 of max(1, |score|) (fp32
logits and exponentials against fp64: the measured error is a few 1e-6); its HRM
flags must match except where two blocks hold a row's maximum within fp32 rounding
of the logits.  Every mask row is compared with the oracle's: it must be ordered by
(HRM flag, oracle score) descending and hold the oracle's kept set, where two
entries may trade places only if their fp64 scores are within that tolerance of
each other (or a flag differs at a flag tie).  The fixed-fraction length is exact;
the Top-p length equals the oracle's or is off by one only where the cumulative
score sits within rounding of the threshold.
"""
import math
import sys

import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from oracle import kap
from tests.parity_helpers import oracle_arrays

pytestmark = pytest.mark.gpu

FLAG_TIE = 1e-4   # a Pbar within this of 1 may be the row maximum on either side
SCORE_TOL = 1e-5  # block scores: |gpu - oracle| <= SCORE_TOL * max(1, |oracle|)


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


def check_row_against_oracle(row, so, flags, n_cand, tol):
    """The GPU's mask row (its kept entries in visit order) against the oracle's scores
    so and the flags the row is ranked by: in (flag desc, score desc) order up to tol,
    and no left-out candidate ranked above a kept one by more than tol.  Returns
    whether the row differs from the exact (flag, score, id) order."""
    ids = np.arange(n_cand)
    exact = ids[np.lexsort((ids, -so, -flags))][: row.size]
    assert len(set(row.tolist())) == row.size and np.all((row >= 0) & (row < n_cand)), "row ids"
    if np.array_equal(row, exact):
        return False
    fa, sa = flags[row], so[row]
    for x in range(row.size - 1):
        assert fa[x] > fa[x + 1] or (fa[x] == fa[x + 1] and sa[x] >= sa[x + 1] - tol), \
            f"order at {x}: ({fa[x]}, {sa[x]}) before ({fa[x + 1]}, {sa[x + 1]})"
    out = np.setdiff1d(ids, row)
    if out.size and row.size:
        # the weakest kept entry against the strongest left-out one
        for f in (0, 1):
            kept_f, out_f = sa[fa == f], so[out][flags[out] == f]
            if out_f.size and kept_f.size:
                assert kept_f.min() >= out_f.max() - tol, "kept set"
        if (flags[out] == 1).any():
            assert (fa == 1).all(), "a flagged candidate was left out while an unflagged one was kept"
    return True


def check_kap(rt, name, batch, stride, mode, budget, blocks=None, sm_scale=None):
    import torch
    Hkv = batch.k_pool.shape[1]
    db = rt.upload(batch)
    om_d, ml_d, sc_d, fl_d = rt.build_kap_mask(db, stride, mode, budget, outputs=True, sm_scale=sm_scale or 0.0)
    torch.cuda.synchronize()
    om_g, ml_g = om_d.cpu().numpy(), ml_d.cpu().numpy()
    sc_g, fl_g = sc_d.cpu().numpy(), fl_d.cpu().numpy()
    q, k, _, pt, B = oracle_arrays(batch)
    nqb = om_g.shape[0]
    want = list(range(nqb)) if blocks is None else list(blocks)
    om_o, ml_o, sc_o, fl_o, hm_o = kap.build_kap_mask(q, k, pt, batch.cu_seqlens, Hkv, stride, mode, budget,
                                                      page_size=B, width=om_g.shape[2], blocks=want,
                                                      return_hmax=True, sm_scale=sm_scale)
    starts = np.cumsum([0] + [-(-int(L) // B) for L in np.diff(batch.cu_seqlens)])
    stats = dict(units=0, flag_ties=0, len_ties=0, rows_reordered=0, max_score_err=0.0, max_score_rel=0.0)
    for pos, qb in enumerate(want):
        sidx = int(np.searchsorted(starts, qb, side="right") - 1)
        i = qb - int(starts[sidx])
        for g in range(Hkv):
            stats["units"] += 1
            so, sg = sc_o[pos, g, : i + 1], sc_g[qb, g, : i + 1]
            scale = np.maximum(1.0, np.abs(so))
            err = np.abs(sg.astype(np.float64) - so)
            stats["max_score_err"] = max(stats["max_score_err"], float(err.max()))
            stats["max_score_rel"] = max(stats["max_score_rel"], float((err / scale).max()))
            assert np.all(err <= SCORE_TOL * scale), f"{name} scores qb {qb} g {g}: {float((err / scale).max())}"
            assert np.all(np.isnan(sc_g[qb, g, i + 1:])) and np.all(fl_g[qb, g, i + 1:] == 0)
            fo, fg = fl_o[pos, g, : i + 1].astype(bool), fl_g[qb, g, : i + 1].astype(bool)
            near = hm_o[pos, g, : i + 1] >= 1.0 - FLAG_TIE
            diff = fo != fg
            if diff.any():
                # only near-maximal blocks may differ, and only in rows with two of them
                assert np.all(near[diff]) and near.sum() >= 2, f"{name} flags qb {qb} g {g}: {np.flatnonzero(diff)}"
                stats["flag_ties"] += int(diff.sum())
            n = int(ml_g[qb, g])
            row = om_g[qb, g]
            assert np.all(row[n:] == -1)
            if mode == kap.MODE_FRACTION:
                assert n == int(ml_o[pos, g])
            elif n != int(ml_o[pos, g]):
                order = np.lexsort((np.arange(i + 1), -so, -fo.astype(np.int64)))
                cs = np.cumsum(so[order])
                thr = np.float32(budget) * so.sum()
                k = int(ml_o[pos, g])
                assert abs(n - k) == 1, f"{name} top-p length qb {qb} g {g}: {n} vs {k}"
                edge = cs[min(n, k) - 1]
                assert abs(edge - thr) <= 1e-3 * max(1.0, thr), f"{name} top-p edge qb {qb} g {g}"
                stats["len_ties"] += 1
            # the row against the oracle's scores, ranked by the flags the kernel took
            # (equal to the oracle's except at the flag ties allowed above)
            tol = SCORE_TOL * max(1.0, float(np.max(np.abs(so))))
            try:
                stats["rows_reordered"] += check_row_against_oracle(row[:n].astype(np.int64), so,
                                                                    fg.astype(np.int64), i + 1, 2 * tol)
            except AssertionError as e:
                raise AssertionError(f"{name} row qb {qb} g {g}: {e}") from None
    assert stats["flag_ties"] <= max(2, stats["units"] // 100)
    log(name, stats)
    return stats


SMALL = [
    # name, seq_lens, hq, hkv, generator, pool, stride, mode, budget
    ("gqa4_s16_frac", [64 * 37 + 13, 64 * 5], 8, 2, "structured", "shuffled", 16, kap.MODE_FRACTION, 0.3),
    ("gqa4_s16_topp", [64 * 37 + 13, 64 * 5], 8, 2, "structured", "shuffled", 16, kap.MODE_TOP_P, 0.9),
    ("gqa4_s8_frac", [64 * 20 + 40], 8, 2, "iid", "identity", 8, kap.MODE_FRACTION, 0.5),
    ("gqa4_s8_topp", [64 * 20 + 40], 8, 2, "structured", "identity", 8, kap.MODE_TOP_P, 0.95),
    ("mha_s16", [64 * 30 + 1], 2, 2, "iid", "shuffled", 16, kap.MODE_FRACTION, 0.2),
    ("gqa2_s8", [64 * 9, 64 * 9 + 63, 17], 4, 2, "structured", "shuffled", 8, kap.MODE_TOP_P, 0.8),
    ("gqa8_s16", [64 * 12 + 5], 16, 2, "structured", "identity", 16, kap.MODE_FRACTION, 0.25),
    # an empty and a one-token sequence between ragged ones: no tiles, and one sampled key
    ("edges_s16", [64 * 7 + 3, 0, 1, 64 * 5], 8, 2, "structured", "shuffled", 16, kap.MODE_FRACTION, 0.3),
    ("edges_s8", [64 * 7 + 3, 0, 1, 64 * 5], 8, 2, "structured", "shuffled", 8, kap.MODE_TOP_P, 0.9),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_kap_small(rt, case):
    name, lens, hq, hkv, gen, pool, stride, mode, budget = case
    log("case", name, lens, hq, hkv, gen, pool, stride, mode, budget)
    wl = inputs.small_workload(name, lens, hq, hkv, generator=gen, seed=77, pool=pool)
    check_kap(rt, name, inputs.generate(wl), stride, mode, budget)


@pytest.mark.parametrize("stride,mode,budget", [(16, kap.MODE_FRACTION, 0.3), (8, kap.MODE_TOP_P, 0.9)])
def test_kap_multi_chunk_sequences(rt, stride, mode, budget):
    # a 19K-token sequence spans 38 (stride 16) or 76 (stride 8) key tiles of 32 samples:
    # its query groups split their keys over two or three chunks whose row maxima combine
    # in the workspace; the sequences around it put its tiles and the next sequence's at
    # nonzero slots
    lens = [64 * 9, 64 * 300 + 17, 64 * 40 + 5]
    log("case multi-chunk", lens, "stride", stride, "mode", mode, "budget", budget)
    wl = inputs.small_workload(f"chunks_s{stride}", lens, 4, 2, generator="structured", seed=91, pool="shuffled")
    check_kap(rt, f"multi-chunk s{stride}", inputs.generate(wl), stride, mode, budget)


def test_kap_rejects_unsupported(rt):
    import torch
    from block_sparse_long_osk_amd import binding
    wl = inputs.small_workload("rej", [64 * 3], 12, 4, generator="iid", seed=1, pool="identity")  # G = 3
    db = rt.upload(inputs.generate(wl))
    with pytest.raises(binding.CosaError):
        rt.build_kap_mask(db, 16, kap.MODE_FRACTION, 0.5)
    wl = inputs.small_workload("rej2", [64 * 3], 8, 2, generator="iid", seed=1, pool="identity")
    db = rt.upload(inputs.generate(wl))
    with pytest.raises(binding.CosaError):
        rt.build_kap_mask(db, 32, kap.MODE_FRACTION, 0.5)         # stride 32: not supported
    with pytest.raises(binding.CosaError):
        rt.build_kap_mask(db, 16, 7, 0.5, width=8)                 # unknown mode
    torch.cuda.synchronize()


def test_kap_full_size_128k_sampled(rt):
    wl = inputs.WORKLOADS["cfg4_128k_structured"]
    batch = inputs.generate(wl)
    rng = np.random.default_rng(5)
    blocks = sorted(set([0, 1, 2047] + rng.choice(2048, 24, replace=False).tolist()))
    log("cfg4 KAP sampled blocks", blocks)
    check_kap(rt, "cfg4_kap_frac", batch, 16, kap.MODE_FRACTION, 0.1, blocks=blocks)
    check_kap(rt, "cfg4_kap_topp", batch, 16, kap.MODE_TOP_P, 0.95, blocks=blocks[:12])
