"""Pins of the oracles on page-table entries that name no page of the physical pool.

PageWeaver notes, section 2.1 (conventions): an id that does not name a stored
page adds no interaction.  A page-table entry of -1 (an unmapped page) or one at
or past the pool size therefore makes its logical page unusable:

* the prefill oracle and brute force do not visit it -- the result equals that of
  the same mask with those entries removed, and the entries are logged as not
  visited (code 2, margin NaN);
* the mean-pooled and KAP builders see no stored keys there -- the result equals
  that of a pool holding an explicit all-zero page for it.

Each expected value comes from a run with no unusable entry at all, so a mistake in
the oracles' handling of such entries (reading the pool at a negative index, or
visiting the page) fails here.
"""
import math

import numpy as np
import pytest

from oracle import kap, maskref, osk
from tests.oracle_helpers import make_problem, random_masks

D = 16
P = 16


def _problem(seed):
    rng = np.random.default_rng(seed)
    lens = [P * 6 + 5, P * 4]
    q, k, v, pt, cu = make_problem(rng, lens, 4, 2, D, P, shuffled=True, scale=1.5)
    om, ml = random_masks(rng, lens, 2, P, 9, junk=False, full_fraction=1.0)
    return rng, lens, q, k, v, pt, cu, om, ml


def _remove_ids(om, ml, cu_qb, drop):
    """The same rows with every entry naming (sequence, logical id) in drop removed;
    also returns, per row, the position each kept entry moves to."""
    om2 = np.full_like(om, -1)
    ml2 = np.zeros_like(ml)
    pos = np.full(om.shape, -1, dtype=np.int64)
    for qb in range(om.shape[0]):
        s = int(np.searchsorted(cu_qb, qb, side="right") - 1)
        for g in range(om.shape[1]):
            n = 0
            for kk in range(int(ml[qb, g])):
                j = int(om[qb, g, kk])
                if (s, j) in drop:
                    continue
                om2[qb, g, n] = j
                pos[qb, g, kk] = n
                n += 1
            ml2[qb, g] = n
    return om2, ml2, pos


@pytest.mark.parametrize("bad_value", [-1, "past_pool"])
def test_prefill_oracle_does_not_visit_unmapped_pages(bad_value):
    rng, lens, q, k, v, pt, cu, om, ml = _problem(23)
    n_phys = k.shape[0]
    cu_qb = np.concatenate([[0], np.cumsum([-(-L // P) for L in lens])])
    bad = -1 if bad_value == -1 else n_phys + 3
    pt_bad = pt.copy()
    pt_bad[0, 2] = bad
    pt_bad[1, 1] = bad
    om2, ml2, pos = _remove_ids(om, ml, cu_qb, {(0, 2), (1, 1)})
    assert (ml2 < ml).any()
    delta = float(max(lens) * math.exp(-0.3))
    got = osk.osk_reference(q, k, v, pt_bad, cu, om, ml, delta=delta, page_size=P)
    ref = osk.osk_reference(q, k, v, pt, cu, om2, ml2, delta=delta, page_size=P)
    assert (ref["decisions"] == osk.NOT_COMPUTED_SKIP).any()
    np.testing.assert_allclose(got["out"], ref["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"], ref["lse"], rtol=0, atol=1e-12)
    # every entry naming an unusable page is logged as not visited; the others keep
    # the decision and margin they have in the run without those entries
    G = q.shape[1] // k.shape[1]
    for qb in range(om.shape[0]):
        for h in range(q.shape[1]):
            g = h // G
            for kk in range(int(ml[qb, g])):
                if pos[qb, g, kk] < 0:
                    assert got["decisions"][qb, h, kk] == osk.NOT_VISITED
                    assert np.isnan(got["margins"][qb, h, kk])
                else:
                    assert got["decisions"][qb, h, kk] == ref["decisions"][qb, h, pos[qb, g, kk]]
                    assert got["margins"][qb, h, kk] == pytest.approx(ref["margins"][qb, h, pos[qb, g, kk]],
                                                                      abs=1e-12)
    # brute force over the support sets agrees, and so does the run without skipping
    bf_got = osk.brute_force_attention(q, k, v, pt_bad, cu, om, ml, page_size=P)
    bf_ref = osk.brute_force_attention(q, k, v, pt, cu, om2, ml2, page_size=P)
    np.testing.assert_allclose(bf_got[0], bf_ref[0], rtol=0, atol=1e-12)
    off = osk.osk_reference(q, k, v, pt_bad, cu, om, ml, delta=-1.0, page_size=P)
    np.testing.assert_allclose(off["out"], bf_ref[0], rtol=0, atol=1e-12)


def _with_zero_page(k, pt, where):
    """The pool with one extra all-zero page, and the page table pointing the
    (sequence, logical page) pairs in `where` at it."""
    kz = np.concatenate([k, np.zeros_like(k[:1])], axis=0)
    ptz = pt.copy()
    for s, j in where:
        ptz[s, j] = k.shape[0]
    return kz, ptz


@pytest.mark.parametrize("bad_value", [-1, "past_pool"])
def test_mean_pooled_builder_sees_zero_keys_on_unmapped_pages(bad_value):
    _, lens, q, k, v, pt, cu, _, _ = _problem(29)
    bad = -1 if bad_value == -1 else k.shape[0] + 7
    pt_bad = pt.copy()
    pt_bad[0, 3] = bad
    kz, ptz = _with_zero_page(k, pt, [(0, 3)])
    got = maskref.build_order_mask(q, k, pt_bad, cu, 2, 0.5, page_size=P, return_scores=True)
    ref = maskref.build_order_mask(q, kz, ptz, cu, 2, 0.5, page_size=P, return_scores=True)
    for x, y in zip(got, ref):
        np.testing.assert_array_equal(np.nan_to_num(x, nan=-7.0), np.nan_to_num(y, nan=-7.0))
    # the unmapped page scores exactly 0 in every row of its sequence that can see it
    sc = got[2]
    assert np.all(sc[3:7, :, 3] == 0.0)
    unions = maskref.build_union_mask(q, k, pt_bad, cu, 2, 0.5, page_size=P)
    unions_z = maskref.build_union_mask(q, kz, ptz, cu, 2, 0.5, page_size=P)
    for x, y in zip(unions, unions_z):
        np.testing.assert_array_equal(np.asarray(x), np.asarray(y))


@pytest.mark.parametrize("mode,budget", [(kap.MODE_FRACTION, 0.5), (kap.MODE_TOP_P, 0.9)])
def test_kap_builder_sees_zero_keys_on_unmapped_pages(mode, budget):
    _, lens, q, k, v, pt, cu, _, _ = _problem(37)
    pt_bad = pt.copy()
    pt_bad[0, 4] = -1
    pt_bad[1, 0] = k.shape[0] + 1
    kz, ptz = _with_zero_page(k, pt, [(0, 4), (1, 0)])
    got = kap.build_kap_mask(q, k, pt_bad, cu, 2, 4, mode, budget, page_size=P)
    ref = kap.build_kap_mask(q, kz, ptz, cu, 2, 4, mode, budget, page_size=P)
    for x, y in zip(got, ref):
        np.testing.assert_array_equal(np.nan_to_num(np.asarray(x, dtype=np.float64), nan=-7.0),
                                      np.nan_to_num(np.asarray(y, dtype=np.float64), nan=-7.0))
