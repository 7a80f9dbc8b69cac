"""Comparison of the HIP path against the fp64 oracle (used by the GPU tests).

Bars (BASELINE the benchmark spec): output max-abs error <= 1e-2 and relative Frobenius
error <= 5e-3 against the oracle on bf16 inputs; skip decisions identical except
where the oracle's margin is within 1e-3 of the threshold (counted, and then the
GPU's choice is followed); "not visited" codes identical.  Margins and LSE are
fp32 quantities of O(1): they are held to 1e-4 (margins, + 1e-5 relative) and
2e-3 (LSE, which also carries the bf16 rounding of P in its sum) -- well above
fp32 accumulation error over 128-term dot products, well below any decision- or
support-changing difference.
"""
import math

import numpy as np

from block_sparse_long_osk_amd import inputs
from oracle import decision_fixture, paging
from oracle.osk import NOT_VISITED, ReplayDecisions, block_thresholds, osk_reference

MAX_ABS = 1e-2
REL_FROB = 5e-3
MARGIN_ABS = 1e-4
MARGIN_REL = 1e-5
LSE_ABS = 2e-3


def host_arrays(batch):
    return (inputs.bf16_bits_to_f32(batch.q), inputs.bf16_bits_to_f32(batch.k_pool),
            inputs.bf16_bits_to_f32(batch.v_pool))


def oracle_arrays(batch):
    """(q, k, v, page_table, B): float arrays with the pools at the batch's logical block
    size B (the oracle's view when physical pages are smaller or larger than B)."""
    q, k, v = host_arrays(batch)
    B, P = batch.block_size, k.shape[2]
    pt = batch.page_table
    if P != B:
        k, v, pt = paging.logical_view(k, v, pt, batch.cu_seqlens, P, block=B)
    return q, k, v, pt, B


def gpu_to_host(outputs):
    res = {"out": outputs.out.float().cpu().numpy(), "lse": outputs.lse.cpu().numpy()}
    if outputs.decisions is not None:
        res["decisions"] = outputs.decisions.cpu().numpy()
        res["margins"] = outputs.margins.cpu().numpy()
    return res


def unit_rows(batch, units):
    """Token rows [T] bool and (qb, head) pairs covered by units (qb, g)."""
    Hq, Hkv = batch.q.shape[1], batch.k_pool.shape[1]
    G = Hq // Hkv
    rows = np.zeros((batch.q.shape[0], Hq), dtype=bool)
    cu_qb, cu, B = batch.cu_qblocks, batch.cu_seqlens, batch.block_size
    for qb, g in units:
        s = int(np.searchsorted(cu_qb, qb, side="right") - 1)
        i = qb - cu_qb[s]
        t0 = cu[s] + B * i
        t1 = min(cu[s + 1], t0 + B)
        rows[t0:t1, g * G:(g + 1) * G] = True
    return rows


def check_prefill(batch, order_mask, mask_len, delta, gpu, units=None, require_log=True, membership=None,
                  sm_scale=None):
    """Oracle replay vs the GPU result; returns a stats dict, asserts the bars.
    membership: the per-q-head membership of the union rows (None: shared rows)."""
    q, k, v, pt, B = oracle_arrays(batch)
    Hq, Hkv = q.shape[1], k.shape[1]
    if units is None:
        units = [(qb, g) for qb in range(batch.total_qblocks) for g in range(Hkv)]
    taus = block_thresholds(batch.cu_seqlens, delta, page_size=B)
    rep = ReplayDecisions(gpu["decisions"], taus) if "decisions" in gpu else None
    ref = osk_reference(q, k, v, pt, batch.cu_seqlens, order_mask, mask_len, delta, page_size=B,
                        units=units, decision_override=rep, membership=membership, sm_scale=sm_scale)
    stats = {"units": len(units)}
    rows = unit_rows(batch, units)
    # ---- decisions and margins
    if rep is not None:
        evaluated = ref["decisions"] != 255
        gd, rd = gpu["decisions"], ref["decisions"]
        nv_mismatch = int(((rd == NOT_VISITED) != (gd == NOT_VISITED))[evaluated].sum())
        stats.update(near_ties=rep.near_ties, near_tie_flips=rep.near_tie_flips,
                     disagreements=len(rep.disagreements), not_visited_mismatch=nv_mismatch,
                     visited=int((evaluated & (rd != NOT_VISITED)).sum()),
                     skipped=int((evaluated & (rd == 1)).sum()))
        assert nv_mismatch == 0, "visit sets differ"
        assert not rep.disagreements, f"decisions differ away from the threshold: {rep.disagreements[:5]}"
        vis = evaluated & (rd != NOT_VISITED)
        gm, rm = gpu["margins"][vis], ref["margins"][vis]
        fin = np.isfinite(rm)
        assert np.array_equal(fin, np.isfinite(gm))
        err = np.abs(gm[fin] - rm[fin])
        stats["margin_max_err"] = float(err.max()) if err.size else 0.0
        assert (err <= MARGIN_ABS + MARGIN_REL * np.abs(rm[fin])).all(), stats["margin_max_err"]
        assert np.isnan(gpu["margins"][evaluated & (rd == NOT_VISITED)]).all()
        # a head's first visit moves every row's running max from -inf to m_loc: its
        # margin is exactly 0 (no rounding residue of the logit scaling)
        gvis = gd != NOT_VISITED
        has = gvis.any(axis=2)
        first = np.take_along_axis(gpu["margins"], gvis.argmax(axis=2)[..., None], axis=2)[..., 0]
        assert (first[has] == 0.0).all(), "first-visit margins are not exactly 0"
    elif require_log:
        raise AssertionError("decision log required")
    # ---- output
    go, ro = gpu["out"][rows], ref["out"][rows]
    diff = np.abs(go - ro)
    stats["max_abs"] = float(diff.max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ro))
    stats["rel_frob"] = float(np.linalg.norm(go - ro) / nrm) if nrm > 0 else float(np.linalg.norm(go))
    assert stats["max_abs"] <= MAX_ABS, stats
    assert stats["rel_frob"] <= REL_FROB, stats
    # worst (head, block) by relative error
    worst = (0.0, None)
    cu_qb = batch.cu_qblocks
    for qb, g in units[: 4096]:
        s = int(np.searchsorted(cu_qb, qb, side="right") - 1)
        t0 = batch.cu_seqlens[s] + B * (qb - cu_qb[s])
        t1 = min(batch.cu_seqlens[s + 1], t0 + B)
        G = Hq // Hkv
        for h in range(g * G, (g + 1) * G):
            a, b = gpu["out"][t0:t1, h], ref["out"][t0:t1, h]
            n = np.linalg.norm(b)
            e = np.linalg.norm(a - b) / n if n > 0 else np.linalg.norm(a)
            if e > worst[0]:
                worst = (float(e), (int(qb), int(h)))
    stats["worst_block_rel"] = worst[0]
    stats["worst_block"] = worst[1]
    # ---- LSE
    gl, rl = gpu["lse"][rows], ref["lse"][rows]
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(gl)), "empty-support rows differ"
    stats["lse_max_err"] = float(np.abs(gl[fin] - rl[fin]).max()) if fin.any() else 0.0
    assert stats["lse_max_err"] <= LSE_ABS, stats
    return stats


def delta_for_skip_fraction(batch, order_mask, mask_len, fraction=0.4, membership=None, sm_scale=None):
    """A skip scale giving about `fraction` skipped visits on this batch, from the
    oracle's own (decision-independent) margins.  The threshold is put in the middle of
    a gap of at least 2e-3 between consecutive distinct margins (the split nearest the
    fraction), so that no margin is a near-tie and every decision is held exactly;
    without such a gap, at the plain quantile."""
    q, k, v, pt, B = oracle_arrays(batch)
    ref = osk_reference(q, k, v, pt, batch.cu_seqlens, order_mask, mask_len, -1.0, page_size=B,
                        compute_output=False, membership=membership, sm_scale=sm_scale)
    m = ref["margins"]
    lnL = np.zeros(m.shape[0])
    for s in range(len(batch.cu_seqlens) - 1):
        L = int(batch.cu_seqlens[s + 1] - batch.cu_seqlens[s])
        if L > 0:  # an empty sequence has no query blocks
            lnL[batch.cu_qblocks[s]:batch.cu_qblocks[s + 1]] = math.log(L)
    x = np.sort((m + lnL[:, None, None])[np.isfinite(m)])
    kq = int(round(fraction * x.size))
    splits = np.flatnonzero(np.diff(x) > 2e-3) + 1      # x[k-1] < x[k] - 2e-3
    if splits.size:
        kq = int(splits[np.argmin(np.abs(splits - fraction * x.size))])
    return float(math.exp(0.5 * (x[kq - 1] + x[kq])))


def check_mask_against_reference(gpu_om, gpu_ml, ref_om, ref_ml, ref_scores, rel_tol=1e-5):
    """GPU builder vs the fp64 reference: rows equal, or differing only among pages
    whose fp64 scores are within rel_tol (of the row's largest |score|) of each other."""
    assert np.array_equal(gpu_ml, ref_ml), "row lengths differ"
    differ = 0
    nq, hkv, _ = ref_om.shape
    for qb in range(nq):
        for g in range(hkv):
            n = ref_ml[qb, g]
            a, b = gpu_om[qb, g, :n], ref_om[qb, g, :n]
            assert (gpu_om[qb, g, n:] == -1).all()
            if np.array_equal(a, b):
                continue
            differ += 1
            sc = ref_scores[qb, g]
            tol = rel_tol * float(np.nanmax(np.abs(sc))) + 1e-9
            # same forced pages, distinct causal ids
            assert len(set(a.tolist())) == n and all(0 <= x < sc.size and np.isfinite(sc[x]) for x in a)
            sa, sb = sc[a], sc[b]
            # kept sets differ only across near-equal scores
            only_a = sorted(set(a.tolist()) - set(b.tolist()))
            only_b = sorted(set(b.tolist()) - set(a.tolist()))
            if only_a:
                assert abs(sc[only_a].min() - sc[only_b].max()) <= tol or sc[only_a].min() >= sc[only_b].max() - tol
            # order: non-increasing scores up to the tolerance
            assert (np.diff(sa) <= tol).all(), (qb, g)
    return differ


def check_full_decision_log(name, order_mask, mask_len, num_q_heads, gpu_decisions):
    """Every visit's skip decision against the fp64 oracle's, stored for the full-size
    workload by oracle/decision_fixture.py (CoSA section 3.3, Eq. (5)).

    order_mask / mask_len: the oracle's mask the GPU ran (rebuilt by the test); the
    stored per-row CRCs say which rows equal the ones the fixture was made from
    (all of them unless the host's BLAS rounds a proxy score differently at a tie).
    Decisions must be identical except where the oracle's margin is within 1e-3 of
    the threshold; entries past a row's length must be logged as not visited."""
    fx = decision_fixture.load(name)
    nqb, hkv, width = order_mask.shape
    G = num_q_heads // hkv
    assert np.array_equal(np.asarray(mask_len, dtype=np.int32), fx["mask_len"]), "row lengths differ"
    same_rows = decision_fixture.row_crcs(order_mask, mask_len) == fx["row_crc"]
    visited = np.arange(width)[None, None, :] < np.repeat(mask_len, G, axis=1)[:, :, None]
    assert visited.sum() == fx["n"]
    gd = np.asarray(gpu_decisions)
    assert gd.shape == (nqb, num_q_heads, width)
    assert np.all(gd[~visited] == NOT_VISITED), "entries past the row length were visited"
    g_vis = gd[visited]
    assert np.all((g_vis == 0) | (g_vis == 1)), "a mask entry of a canonical row was not visited"
    rows_ok = np.broadcast_to(np.repeat(same_rows, G, axis=1)[:, :, None], visited.shape)[visited]
    differ = (g_vis == 1) != fx["skip"]
    stats = dict(visits=int(fx["n"]), compared=int(rows_ok.sum()), rows_not_matching_fixture=int((~same_rows).sum()),
                 skipped=int((g_vis == 1).sum()), near_ties=int((fx["near"] & rows_ok).sum()),
                 near_tie_flips=int((differ & fx["near"] & rows_ok).sum()),
                 disagreements=int((differ & ~fx["near"] & rows_ok).sum()))
    assert stats["rows_not_matching_fixture"] <= max(1, same_rows.size // 1000), stats
    assert stats["disagreements"] == 0, stats
    return stats
