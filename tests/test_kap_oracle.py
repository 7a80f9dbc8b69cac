"""Pins of the KAP oracle (CoSA section 4.2, Eq. (8)-(14); Appendix C, Figure A and
Algorithm A, pre-kernel proxy) against facts that do not come from the oracle's own
formula: the closed form that MaxNorm leaves (the softmax normaliser cancels), a
library argmax for the HRM flags, causality and stride invariance, and the ordering
and selection properties Eq. (13)-(14) define."""
import math

import numpy as np
import pytest

from oracle import kap

P = 64
D = 128


def rand_case(L, hq, hkv, seed, pages=None):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((L, hq, D)) / math.sqrt(D)).astype(np.float32)
    n = -(-L // P)
    k_pool = rng.standard_normal((n, hkv, P, D)).astype(np.float32)
    pt = np.arange(n, dtype=np.int32)[None, :] if pages is None else pages
    return q, k_pool, pt, np.array([0, L], dtype=np.int64)


def raw_scores(q, k_pool, pt, h, g, stride, L):
    """x[r, c] = q~_r . k~_c over sampled tokens, straight from the inputs (float64)."""
    toks = np.arange(0, L, stride)
    qs = q[toks, h, :].astype(np.float64)
    ks = np.stack([k_pool[pt[0][t // P], g, t % P, :] for t in toks]).astype(np.float64)
    return qs @ ks.T


def test_one_sample_per_block_is_exp_of_score_gap():
    # stride = block size: block j holds one sampled key; MaxPool is the identity and
    # MaxNorm divides the softmax by its row maximum, so Pbar[i, j] = exp((x_ij - max_j' x_ij') / sqrt(d))
    L = 64 * 9
    q, k, pt, cu = rand_case(L, 1, 1, 3)
    _, _, sc, fl = kap.build_kap_mask(q, k, pt, cu, 1, 64, kap.MODE_FRACTION, 1.0)
    x = raw_scores(q, k, pt, 0, 0, 64, L)
    for i in range(9):
        xi = x[i, : i + 1]
        want = np.exp((xi - xi.max()) / math.sqrt(D))
        np.testing.assert_allclose(sc[i, 0, : i + 1], want, rtol=1e-12, atol=1e-15)
        assert np.argmax(xi) == int(np.flatnonzero(fl[i, 0, : i + 1])[0])
        assert fl[i, 0, : i + 1].sum() == 1


def test_caller_scale_replaces_inverse_sqrt_d():
    # the same one-sample-per-block closed form with a caller's logit scale s in place
    # of 1/sqrt(d): Pbar[i, j] = exp(s (x_ij - max_j' x_ij')); s = 1/sqrt(d) is the default
    L = 64 * 7
    q, k, pt, cu = rand_case(L, 1, 1, 5)
    x = raw_scores(q, k, pt, 0, 0, 64, L)
    s = 0.25
    _, _, sc, _ = kap.build_kap_mask(q, k, pt, cu, 1, 64, kap.MODE_FRACTION, 1.0, sm_scale=s)
    for i in range(7):
        xi = x[i, : i + 1]
        np.testing.assert_allclose(sc[i, 0, : i + 1], np.exp(s * (xi - xi.max())), rtol=1e-12, atol=1e-15)
    _, _, a, _ = kap.build_kap_mask(q, k, pt, cu, 1, 64, kap.MODE_FRACTION, 1.0)
    _, _, b, _ = kap.build_kap_mask(q, k, pt, cu, 1, 64, kap.MODE_FRACTION, 1.0, sm_scale=1.0 / math.sqrt(D))
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=0)


@pytest.mark.parametrize("stride", [16, 8])
def test_hrm_flags_are_the_blocks_holding_row_maxima(stride):
    L, hq, hkv = 64 * 7 + 20, 4, 2
    q, k, pt, cu = rand_case(L, hq, hkv, 11)
    _, _, sc, fl = kap.build_kap_mask(q, k, pt, cu, hkv, stride, kap.MODE_FRACTION, 1.0)
    per = P // stride
    G = hq // hkv
    for g in range(hkv):
        xs = [raw_scores(q, k, pt, g * G + hh, g, stride, L) for hh in range(G)]
        R = xs[0].shape[0]
        for i in range(-(-L // P)):
            want = set()
            for x in xs:
                for r in range(i * per, min((i + 1) * per, R)):
                    want.add(int(np.argmax(x[r, : r + 1])) // per)   # block of the row's argmax
            got = set(np.flatnonzero(fl[i, g, : i + 1]).tolist())
            assert got == want, (g, i)
            rows = min((i + 1) * per, R) - i * per
            # every sampled row of every head puts exactly 1 into its argmax block and less elsewhere
            assert np.all(sc[i, g, : i + 1] <= G * rows + 1e-12)
            assert sc[i, g, list(want)].sum() >= G * rows - 1e-9
            assert np.all(sc[i, g, : i + 1] >= 0)


def test_causal_and_stride_invariance():
    L, stride = 64 * 6, 16
    q, k, pt, cu = rand_case(L, 4, 1, 5)
    base = kap.build_kap_mask(q, k, pt, cu, 1, stride, kap.MODE_FRACTION, 0.5)
    # keys of later blocks: invisible to block 2's sampled rows
    k2 = k.copy()
    k2[3:] = np.random.default_rng(9).standard_normal(k2[3:].shape)
    other = kap.build_kap_mask(q, k2, pt, cu, 1, stride, kap.MODE_FRACTION, 0.5)
    for a, b in zip(base, other):
        np.testing.assert_array_equal(np.asarray(a)[:3], np.asarray(b)[:3])
    # tokens that are not sampled (t % stride != 0) in queries and keys: no effect at all
    q3, k3 = q.copy(), k.copy()
    rng = np.random.default_rng(10)
    mask_t = (np.arange(L) % stride) != 0
    q3[mask_t] = rng.standard_normal(q3[mask_t].shape)
    k3[:, :, mask_t[:P], :] = rng.standard_normal(k3[:, :, mask_t[:P], :].shape)
    third = kap.build_kap_mask(q3, k3, pt, cu, 1, stride, kap.MODE_FRACTION, 0.5)
    for a, b in zip(base, third):
        np.testing.assert_array_equal(a, b)


def test_paged_pool_matches_identity_layout():
    L = 64 * 5 + 7
    q, k, pt, cu = rand_case(L, 4, 2, 21)
    n = k.shape[0]
    perm = np.random.default_rng(4).permutation(n + 3)
    pool = np.zeros((n + 3, 2, P, D), dtype=np.float32)
    pool[perm[:n]] = k
    a = kap.build_kap_mask(q, k, pt, cu, 2, 16, kap.MODE_TOP_P, 0.9)
    b = kap.build_kap_mask(q, pool, perm[:n][None, :].astype(np.int32), cu, 2, 16, kap.MODE_TOP_P, 0.9)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("mode,budget", [(kap.MODE_FRACTION, 0.3), (kap.MODE_FRACTION, 0.1),
                                         (kap.MODE_TOP_P, 0.95), (kap.MODE_TOP_P, 0.5)])
def test_order_and_selection(mode, budget):
    L = 64 * 12 + 33
    q, k, pt, cu = rand_case(L, 4, 2, 7)
    om, ml, sc, fl = kap.build_kap_mask(q, k, pt, cu, 2, 16, mode, budget)
    for i in range(om.shape[0]):
        for g in range(2):
            s, h = sc[i, g, : i + 1], fl[i, g, : i + 1]
            full = sorted(range(i + 1), key=lambda j: (-int(h[j]), -s[j], j))
            n = ml[i, g]
            row = om[i, g]
            assert list(row[:n]) == full[:n]                       # HRM first, score desc, id asc
            assert np.all(row[n:] == -1)
            if mode == kap.MODE_FRACTION:
                assert n == max(1, min(i + 1, math.ceil(np.float32(budget) * (i + 1) - 1e-3)))
            else:
                cs = np.cumsum(s[full])
                need = np.float32(budget) * s.sum()
                assert cs[n - 1] >= need and (n == 1 or cs[n - 2] < need)


def test_planted_key_is_visited_first():
    # one key far along the query direction of block 5's rows makes block 2 that
    # block's only HRM block and its top score
    L, stride = 64 * 8, 16
    q, k, pt, cu = rand_case(L, 1, 1, 13)
    u = np.random.default_rng(1).standard_normal(D)
    u /= np.linalg.norm(u)
    q[5 * 64: 6 * 64, 0, :] = (u * 2.0).astype(np.float32)
    k[2, 0, 16, :] = (u * 40.0).astype(np.float32)   # token 2*64+16: a sampled key of block 2
    om, ml, sc, fl = kap.build_kap_mask(q, k, pt, cu, 1, stride, kap.MODE_FRACTION, 0.3)
    assert om[5, 0, 0] == 2
    assert list(np.flatnonzero(fl[5, 0, :6])) == [2]


def test_mask_width_covers_every_row():
    for mode, b in [(kap.MODE_FRACTION, 0.1), (kap.MODE_FRACTION, 0.55), (kap.MODE_TOP_P, 0.9)]:
        for mp in (1, 2, 7, 64, 2048):
            w = kap.mask_width(mp, mode, b)
            if mode == kap.MODE_FRACTION:
                assert w == max(kap.keep_count(mode, b, np.ones(i + 1)) for i in range(mp))
            else:
                assert w == mp


def test_selection_counts_on_exact_values():
    # Top-p: the smallest prefix of the sorted order whose scores reach p of the total
    s = np.array([2.0, 1.0, 1.0])
    assert kap.keep_count(kap.MODE_TOP_P, 0.5, s) == 1      # 2 >= 0.5 * 4 exactly
    assert kap.keep_count(kap.MODE_TOP_P, 0.75, s) == 2     # 3 >= 3 exactly
    assert kap.keep_count(kap.MODE_TOP_P, 0.76, s) == 3
    assert kap.keep_count(kap.MODE_TOP_P, 0.0, s) == 1      # at least one block
    # fixed fraction: 0.1 * 30 rounds to 3.0000000000000004 in binary; the row keeps 3
    assert kap.keep_count(kap.MODE_FRACTION, 0.1, np.ones(30)) == 3
    assert kap.keep_count(kap.MODE_FRACTION, 0.1, np.ones(31)) == 4
    assert kap.keep_count(kap.MODE_FRACTION, 0.1, np.ones(1)) == 1
