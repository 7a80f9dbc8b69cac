"""Pins of the CPU oracle to facts the pages and the mathematics fix (no GPU).

Each test names what it pins.  A plausible slip in the oracle (a dropped
causal cut, a wrong running-max update, the skip test taken after instead of
before the max update, a wrong threshold unit, double-counted repeats) fails at
least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import osk
from oracle.osk import (COMPUTED, NOT_COMPUTED_SKIP, NOT_VISITED, ReplayDecisions,
                        block_thresholds, brute_force_attention, full_causal_mask,
                        osk_reference, support_set)
from tests.oracle_helpers import make_problem, random_masks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- support set
def test_support_set_worked_example():
    """PageWeaver notes 2.1: P=4, S={0,2}, L=11, c=9 -> {0,1,2,3,8,9}."""
    with open(os.path.join(GOLDEN, "support_set_worked_example.json")) as f:
        ex = json.load(f)
    got = support_set(ex["selected_pages"], ex["page_size"], ex["valid_len"], ex["causal_pos"])
    assert got == ex["support"]


def test_support_set_conventions():
    """Invalid ids add nothing, duplicates add no mass, empty support is empty."""
    assert support_set([0, 2, 2, -1, 3, 99], 4, 11, 9) == [0, 1, 2, 3, 8, 9]
    assert support_set([], 4, 11, 9) == []
    assert support_set([2], 4, 11, 7) == []              # page after the query
    assert support_set([2], 4, 9, 10) == [8]             # valid-length cut on the tail page


def test_empty_support_gives_zero_output():
    rng = np.random.default_rng(0)
    q, k, v, pt, cu = make_problem(rng, [10], 2, 1, 8, 4)
    om = np.full((3, 1, 2), -1)
    ml = np.zeros((3, 1), dtype=np.int64)
    ml[1, 0] = 2                                          # only junk entries
    out, lse = brute_force_attention(q, k, v, pt, cu, om, ml, page_size=4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=4)
    assert np.all(res["out"] == 0) and np.all(np.isneginf(res["lse"]))
    assert np.all(res["decisions"] == NOT_VISITED)


# ---------------------------------------------------------------- brute force
def _textbook_causal(q, k, v, scale):
    """softmax(q k^T * scale + causal) v, written out in numpy (fp64)."""
    T = q.shape[0]
    s = (q @ k.T) * scale
    s[np.triu_indices(T, 1)] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w @ v) / w.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("L,P", [(12, 4), (37, 8), (64, 16)])
def test_brute_force_full_mask_is_causal_softmax(L, P):
    """A full causal page set reduces to textbook causal attention, also checked
    against torch's scaled_dot_product_attention in fp64 (a library routine)."""
    rng = np.random.default_rng(L)
    Hq, Hkv, d = 4, 2, 16
    q, k, v, pt, cu = make_problem(rng, [L], Hq, Hkv, d, P, shuffled=True)
    om, ml = full_causal_mask(cu, Hkv, page_size=P)
    out, lse = brute_force_attention(q, k, v, pt, cu, om, ml, page_size=P)
    keys = np.concatenate([k[pt[0, j]] for j in range(-(-L // P))], axis=1)[:, :L]   # [Hkv, L, d]
    vals = np.concatenate([v[pt[0, j]] for j in range(-(-L // P))], axis=1)[:, :L]
    for h in range(Hq):
        ref = _textbook_causal(q[:, h], keys[h // 2], vals[h // 2], 1 / math.sqrt(d))
        np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None], torch.from_numpy(keys[h // 2])[None],
            torch.from_numpy(vals[h // 2])[None], is_causal=True)[0].numpy()
        np.testing.assert_allclose(out[:, h], sdpa, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- online oracle vs brute force
@pytest.mark.parametrize("seed", range(6))
def test_online_matches_brute_force_without_skipping(seed):
    """With skipping off the ordered online softmax equals the softmax over the
    support set (CoSA Eq. (4) order invariance + PageWeaver Eq. (1)-(2)),
    including junk mask entries, ragged tails, packed sequences and GQA."""
    rng = np.random.default_rng(100 + seed)
    P = [2, 4, 8, 16, 4, 8][seed]
    lens = [[9], [13, 5], [31], [40, 17, 64], [1, 8, 3], [16]][seed]
    Hq, Hkv = [(2, 1), (4, 2), (3, 3), (4, 1), (2, 2), (8, 2)][seed]
    d = 8
    q, k, v, pt, cu = make_problem(rng, lens, Hq, Hkv, d, P, shuffled=seed % 2 == 1)
    width = max(-(-L // P) for L in lens) + 4
    om, ml = random_masks(rng, lens, Hkv, P, width)
    out_bf, lse_bf = brute_force_attention(q, k, v, pt, cu, om, ml, page_size=P)
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=P, chunk_blocks=3)
    np.testing.assert_allclose(res["out"], out_bf, rtol=0, atol=1e-12)
    fin = np.isfinite(lse_bf)
    assert np.array_equal(fin, np.isfinite(res["lse"]))
    np.testing.assert_allclose(res["lse"][fin], lse_bf[fin], rtol=0, atol=1e-12)


def test_visit_codes_for_junk_entries():
    """-1, out-of-range, non-causal and repeated ids are 'not visited' (code 2),
    with NaN margins; valid entries are computed when skipping is off."""
    rng = np.random.default_rng(5)
    q, k, v, pt, cu = make_problem(rng, [20], 2, 1, 8, 4)
    om = np.full((5, 1, 6), -1)
    ml = np.zeros((5, 1), dtype=np.int64)
    om[3, 0, :6] = [3, -1, 9, 4, 3, 1]      # block 3 of 5 pages: 9 out of range, 4 non-causal, 3 repeated
    ml[3, 0] = 6
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=4)
    assert list(res["decisions"][3, 0]) == [COMPUTED, NOT_VISITED, NOT_VISITED, NOT_VISITED, NOT_VISITED, COMPUTED]
    assert np.isnan(res["margins"][3, 0, [1, 2, 3, 4]]).all()
    assert res["margins"][3, 0, 0] == 0.0            # the first visit never has a negative margin


def test_order_invariance_without_skipping():
    """CoSA Eq. (4): any permutation of the visit order gives the same output."""
    rng = np.random.default_rng(11)
    lens, P, Hq, Hkv, d = [50, 23], 8, 4, 2, 8
    q, k, v, pt, cu = make_problem(rng, lens, Hq, Hkv, d, P)
    om, ml = full_causal_mask(cu, Hkv, page_size=P)
    base = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=P)
    om2 = om.copy()
    for qb in range(om.shape[0]):
        for g in range(Hkv):
            n = ml[qb, g]
            om2[qb, g, :n] = rng.permutation(om[qb, g, :n])
    perm = osk_reference(q, k, v, pt, cu, om2, ml, delta=-1, page_size=P)
    np.testing.assert_allclose(perm["out"], base["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(perm["lse"], base["lse"], rtol=0, atol=1e-12)


def test_disable_switch():
    """CoSA App. D.1 and the skip test of Algorithm A: Delta = -1 and Delta = 0 both disable the skip."""
    rng = np.random.default_rng(12)
    q, k, v, pt, cu = make_problem(rng, [45], 2, 1, 8, 8, scale=2.0)
    om, ml = full_causal_mask(cu, 1, page_size=8)
    a = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=8)
    b = osk_reference(q, k, v, pt, cu, om, ml, delta=0.0, page_size=8)
    c, _ = brute_force_attention(q, k, v, pt, cu, om, ml, page_size=8)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["decisions"], b["decisions"])
    assert not (a["decisions"] == NOT_COMPUTED_SKIP).any()
    np.testing.assert_allclose(a["out"], c, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed-form skip constructions
def _two_page_construction(a_logit, b_logit, order):
    """d=1, sm_scale=1, P=4, L=8: page 0 keys give logit a to every row, page 1
    keys give logit b; block 1 visits pages in `order`."""
    P, L = 4, 8
    q = np.ones((L, 1, 1))
    k = np.zeros((2, 1, P, 1))
    k[0, 0, :, 0] = a_logit
    k[1, 0, :, 0] = b_logit
    rng = np.random.default_rng(3)
    v = rng.standard_normal((2, 1, P, 1))
    pt = np.array([[0, 1]])
    cu = np.array([0, L])
    om = np.full((2, 1, 2), -1)
    om[0, 0, 0] = 0
    om[1, 0, :] = order
    ml = np.array([[1], [2]])
    return q, k, v, pt, cu, om, ml


@pytest.mark.parametrize("tau,expect_skip", [(-1.0, True), (-3.0, False), (-2.0, False), (-1.999, True)])
def test_skip_rule_closed_form(tau, expect_skip):
    """CoSA Eq. (5): after page 0 (logit 2), page 1 (logit 0) has margin 0 - 2 = -2
    for every row and is skipped iff -2 < tau = ln(Delta/N) (strict).  When
    skipped, each row's output is exactly the mean of page 0's values."""
    q, k, v, pt, cu, om, ml = _two_page_construction(2.0, 0.0, [0, 1])
    delta = 8 * math.exp(tau)
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=4, sm_scale=1.0)
    assert res["margins"][1, 0, 1] == pytest.approx(-2.0, abs=1e-15)
    assert res["decisions"][1, 0, 0] == COMPUTED
    assert res["decisions"][1, 0, 1] == (NOT_COMPUTED_SKIP if expect_skip else COMPUTED)
    o = res["out"][4:8, 0, 0]
    v0 = v[0, 0, :, 0]
    if expect_skip:
        np.testing.assert_allclose(o, np.full(4, v0.mean()), rtol=0, atol=1e-15)
        np.testing.assert_allclose(res["lse"][4:8, 0], np.full(4, 2 + math.log(4)), atol=1e-14)
    else:
        e2 = math.exp(2.0)
        for r in range(4):   # row c = 4 + r sees keys 4..c of page 1
            n1 = r + 1
            ref = (e2 * v0.sum() + v[1, 0, :n1, 0].sum()) / (4 * e2 + n1)
            assert o[r] == pytest.approx(ref, abs=1e-14)


def test_visit_order_changes_what_is_skipped():
    """CoSA Limitation 2: the same pages in ascending order (low page first)
    give margin 0 for the high page (it raises the running max), so nothing is
    skipped; the descending-score order lets the low page be skipped."""
    q, k, v, pt, cu, om, ml = _two_page_construction(0.0, 2.0, [0, 1])
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=8 * math.exp(-1), page_size=4, sm_scale=1.0)
    assert list(res["decisions"][1, 0]) == [COMPUTED, COMPUTED]
    q, k, v, pt, cu, om, ml = _two_page_construction(0.0, 2.0, [1, 0])
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=8 * math.exp(-1), page_size=4, sm_scale=1.0)
    assert list(res["decisions"][1, 0]) == [COMPUTED, NOT_COMPUTED_SKIP]


def test_first_visit_never_skipped_and_delta_above_length_zeroes():
    """tau <= 0 (Delta <= N): the first visit has margin 0 >= tau.  Delta > N makes
    tau > 0, every page skipped, output 0 and LSE -inf (the rule read literally)."""
    rng = np.random.default_rng(21)
    lens = [40]
    q, k, v, pt, cu = make_problem(rng, lens, 2, 1, 8, 8, scale=3.0)
    om, ml = random_masks(rng, lens, 1, 8, 6, junk=False)
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=40.0, page_size=8)
    first = res["decisions"][:, :, 0]
    assert (first == COMPUTED).all()
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=41.0, page_size=8)
    vis = res["decisions"] != NOT_VISITED
    assert (res["decisions"][vis] == NOT_COMPUTED_SKIP).all()
    assert np.all(res["out"] == 0) and np.all(np.isneginf(res["lse"]))


@pytest.mark.parametrize("seed", range(4))
def test_online_with_skip_equals_softmax_over_kept_pages(seed):
    """With skipping on, the result is the softmax restricted to the pages that
    were computed (follows from Alg. A since a skipped page never raises the
    running max when tau <= 0), checked against brute force over that set."""
    rng = np.random.default_rng(300 + seed)
    P = [4, 8, 8, 16][seed]
    lens = [[33], [60, 21], [64], [80]][seed]
    Hq, Hkv = [(2, 1), (4, 2), (2, 2), (4, 1)][seed]
    q, k, v, pt, cu = make_problem(rng, lens, Hq, Hkv, 8, P, scale=1.5)
    width = max(-(-L // P) for L in lens) + 3
    om, ml = random_masks(rng, lens, Hkv, P, width, full_fraction=1.0)
    for frac in (0.35, 0.6, 0.9, 0.99):
        delta = frac * min(lens)
        res = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=P)
        dec = res["decisions"]
        n_skip = int((dec == NOT_COMPUTED_SKIP).sum())
        if n_skip:
            break
    assert n_skip > 0, "construction should skip something"
    kept = {}
    for qb in range(dec.shape[0]):
        for h in range(Hq):
            kept[(qb, h)] = [int(om[qb, h // (Hq // Hkv), kk]) for kk in range(dec.shape[2])
                             if dec[qb, h, kk] == COMPUTED]
    ref, lse = brute_force_attention(q, k, v, pt, cu, om, ml, page_size=P, kept_pages=kept)
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(res["lse"][fin], lse[fin], rtol=0, atol=1e-12)


def test_decisions_do_not_depend_on_value_side():
    """Alg. A updates m before the test whether or not the page is skipped, so the
    logits-only pass yields the same decisions and margins as the full pass."""
    rng = np.random.default_rng(31)
    lens = [70, 30]
    q, k, v, pt, cu = make_problem(rng, lens, 4, 2, 8, 8, scale=1.5)
    om, ml = random_masks(rng, lens, 2, 8, 12)
    full = osk_reference(q, k, v, pt, cu, om, ml, delta=10.0, page_size=8)
    qk = osk_reference(q, k, v, pt, cu, om, ml, delta=10.0, page_size=8, compute_output=False)
    assert np.array_equal(full["decisions"], qk["decisions"])
    np.testing.assert_array_equal(full["margins"], qk["margins"])


def test_threshold_uses_each_sequence_length():
    """tau = ln(Delta / N) with N the sequence's own length (packed batch)."""
    taus = block_thresholds(np.array([0, 128, 192]), delta=32.0, page_size=64)
    assert taus[0] == taus[1] == pytest.approx(math.log(32 / 128))
    assert taus[2] == pytest.approx(math.log(32 / 64))
    assert np.isnan(block_thresholds(np.array([0, 64]), delta=-1.0)).all()


# ---------------------------------------------------------------- replay
def test_replay_of_own_decisions_is_identity():
    rng = np.random.default_rng(41)
    lens = [48]
    q, k, v, pt, cu = make_problem(rng, lens, 2, 1, 8, 8, scale=1.5)
    om, ml = random_masks(rng, lens, 1, 8, 8, junk=False, full_fraction=1.0)
    delta = 15.0
    own = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=8)
    rep = ReplayDecisions(own["decisions"], block_thresholds(cu, delta, 8))
    again = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=8, decision_override=rep)
    assert rep.disagreements == [] and rep.near_tie_flips == 0
    assert np.array_equal(again["out"], own["out"])


def test_replay_flip_at_near_tie_and_disagreement_elsewhere():
    """A decision within 1e-3 of tau may be flipped by the other side and the
    output follows the flipped kept set; a flip far from tau is a disagreement."""
    q, k, v, pt, cu, om, ml = _two_page_construction(2.0, 0.0, [0, 1])
    tau = -2.0 + 5e-4                                   # margin -2 is within 1e-3 below tau: skip
    delta = 8 * math.exp(tau)
    own = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=4, sm_scale=1.0)
    assert own["decisions"][1, 0, 1] == NOT_COMPUTED_SKIP
    other = own["decisions"].copy()
    other[1, 0, 1] = COMPUTED
    rep = ReplayDecisions(other, block_thresholds(cu, delta, 4))
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=4, sm_scale=1.0, decision_override=rep)
    assert rep.near_tie_flips == 1 and rep.disagreements == []
    full = osk_reference(q, k, v, pt, cu, om, ml, delta=-1, page_size=4, sm_scale=1.0)
    np.testing.assert_allclose(res["out"], full["out"], atol=1e-15)
    # far from the threshold the flip is reported and not followed
    delta = 8 * math.exp(-1.0)
    rep = ReplayDecisions(other, block_thresholds(cu, delta, 4))
    res = osk_reference(q, k, v, pt, cu, om, ml, delta=delta, page_size=4, sm_scale=1.0, decision_override=rep)
    assert len(rep.disagreements) == 1 and rep.near_tie_flips == 0
    assert res["decisions"][1, 0, 1] == NOT_COMPUTED_SKIP


def test_empty_sequence_in_a_packed_batch_changes_nothing_else():
    """An empty sequence has no query blocks: packing one between two others leaves their
    outputs, LSE, decisions and margins exactly as without it, and brute force agrees."""
    rng = np.random.default_rng(41)
    lens = [64 * 3 + 9, 70]
    q, k, v, pt, cu = make_problem(rng, lens, 4, 2, 32, 64)
    om, ml = random_masks(rng, lens, 2, 64, 6)
    delta = 100.0
    base = osk.osk_reference(q, k, v, pt, cu, om, ml, delta)
    # the same tokens with an empty sequence in between (its page-table row all -1)
    cu_e = np.array([0, cu[1], cu[1], cu[2]])
    pt_e = np.full((3, pt.shape[1]), -1, dtype=pt.dtype)
    pt_e[0], pt_e[2] = pt[0], pt[1]
    res = osk.osk_reference(q, k, v, pt_e, cu_e, om, ml, delta)
    for key in ("out", "lse", "decisions", "margins"):
        np.testing.assert_array_equal(res[key], base[key])
    np.testing.assert_array_equal(block_thresholds(cu_e, delta), block_thresholds(cu, delta))
    out_bf, _ = osk.brute_force_attention(q, k, v, pt_e, cu_e, om, ml)
    nos = osk.osk_reference(q, k, v, pt_e, cu_e, om, ml, -1.0)
    np.testing.assert_allclose(nos["out"], out_bf, atol=1e-12)
