"""Pins of the CPU mean-pooled-proxy mask reference (no GPU).

The pages print no numeric example of the proxy, so the builder's definition is
a reading (stated in oracle/maskref.py).  What pins its implementation to that
reading: exact keep counts from rational arithmetic, the mask format of CoSA
Eq. (14), and brute-force loops over rows, heads and keys on tiny inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle.maskref import FORCE_DIAG, FORCE_FIRST, build_order_mask, keep_count, mask_width
from tests.oracle_helpers import make_problem


@pytest.mark.parametrize("b1,frac", [(0.5, Fraction(1, 2)), (0.25, Fraction(1, 4)),
                                     (0.2, Fraction(1, 5)), (0.1, Fraction(1, 10))])
def test_keep_count_matches_rational_ceiling(b1, frac):
    for n in range(0, 2100):
        exact = math.ceil(frac * n)
        assert keep_count(float(np.float32(b1)), n) == exact, (b1, n)


def _total_visits(n_pages, frac):
    tot = 0
    for i in range(n_pages):
        nf = 1 if i == 0 else 2
        tot += nf + math.ceil(frac * (i + 1 - nf))
    return tot


@pytest.mark.parametrize("L,frac,visits,width", [
    (2048, Fraction(1, 2), 303, 17),          # 1 head, 2K, 50 %
    (16384, Fraction(1, 4), 8703, 66),        # 16K, 25 %
    (32768, Fraction(1, 5), 27288, 104),      # 32K, 20 %
    (131072, Fraction(1, 10), 214425, 207),   # 128K, 10 %
])
def test_workload_visit_counts(L, frac, visits, width):
    """Row lengths |F_i| + ceil(b1 |R_i|) summed over the blocks of one KV head."""
    n = L // 64
    assert _total_visits(n, frac) == visits
    assert mask_width(n, float(frac)) == width


def _brute_mask(q, k, pt, cu, Hkv, b1, P, flags):
    """Loops over every row, head and key: pooled means, dot products and a
    selection by repeated arg-max with the (score desc, id asc) tie rule."""
    T, Hq, d = q.shape
    G = Hq // Hkv
    rows = []
    for s in range(len(cu) - 1):
        t0, L = int(cu[s]), int(cu[s + 1] - cu[s])
        n = -(-L // P)
        for i in range(n):
            for g in range(Hkv):
                qbar = np.zeros(d)
                for h in range(g * G, (g + 1) * G):
                    acc = np.zeros(d)
                    cnt = 0
                    for r in range(P):
                        c = i * P + r
                        if c < L:
                            acc += q[t0 + c, h]
                            cnt += 1
                    qbar += acc / cnt
                score = {}
                for j in range(i + 1):
                    kacc = np.zeros(d)
                    cnt = 0
                    for t in range(P):
                        if j * P + t < L:
                            kacc += k[pt[s, j], g, t]
                            cnt += 1
                    score[j] = float(qbar @ (kacc / cnt))
                forced = []
                if flags & FORCE_FIRST:
                    forced.append(0)
                if flags & FORCE_DIAG and i not in forced:
                    forced.append(i)
                rest = [j for j in range(i + 1) if j not in forced]
                nk = math.ceil(Fraction(b1).limit_denominator(1000) * len(rest))
                chosen = []
                pool = list(rest)
                for _ in range(nk):
                    best = max(pool, key=lambda j: (score[j], -j))
                    chosen.append(best)
                    pool.remove(best)
                kept = forced + chosen
                kept.sort(key=lambda j: (-score[j], j))
                rows.append(((s, i, g), kept))
    return rows


@pytest.mark.parametrize("seed,lens,Hq,Hkv,b1,flags", [
    (1, [40], 4, 2, 0.5, FORCE_FIRST | FORCE_DIAG),
    (2, [37, 20], 2, 1, 0.25, FORCE_FIRST | FORCE_DIAG),
    (3, [64], 6, 3, 0.2, FORCE_FIRST),
    (4, [50], 4, 4, 0.1, FORCE_DIAG),
    (5, [33], 2, 2, 0.5, 0),
])
def test_builder_matches_brute_force(seed, lens, Hq, Hkv, b1, flags):
    rng = np.random.default_rng(seed)
    P = 4
    q, k, v, pt, cu = make_problem(rng, lens, Hq, Hkv, 6, P, shuffled=True)
    om, ml, sc = build_order_mask(q, k, pt, cu, Hkv, b1, page_size=P, flags=flags, return_scores=True)
    ref = _brute_mask(q, k, pt, cu, Hkv, b1, P, flags)
    qb_of = {}
    qb = 0
    for s, L in enumerate(lens):
        for i in range(-(-L // P)):
            qb_of[(s, i)] = qb
            qb += 1
    for (s, i, g), kept in ref:
        r = qb_of[(s, i)]
        assert ml[r, g] == len(kept)
        assert list(om[r, g, : ml[r, g]]) == kept
        assert (om[r, g, ml[r, g]:] == -1).all()


def test_mask_format_and_gqa_grouping():
    """Eq. (14) format: kept causal ids first, -1 padding after; ids unique;
    permuting the q heads inside a KV group leaves the mask unchanged."""
    rng = np.random.default_rng(9)
    q, k, v, pt, cu = make_problem(rng, [100], 8, 2, 8, 8)
    om, ml = build_order_mask(q, k, pt, cu, 2, 0.3, page_size=8)
    for r in range(om.shape[0]):
        for g in range(2):
            row = om[r, g, : ml[r, g]]
            assert len(set(row.tolist())) == len(row)
            assert (row >= 0).all() and (row <= r).all()
            assert 0 in row and r in row
    q2 = q.copy()
    q2[:, 0:4] = q[:, [2, 0, 3, 1]]
    om2, ml2 = build_order_mask(q2, k, pt, cu, 2, 0.3, page_size=8)
    assert np.array_equal(om, om2) and np.array_equal(ml, ml2)
