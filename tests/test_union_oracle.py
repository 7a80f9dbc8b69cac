"""Pins of the per-q-head page sets under grouped-query heads (PageWeaver notes, section
2.2: the heads of a group traverse the union of their sets, a membership mask keeps
each head's softmax to its own pages; Eq. (3): the logical page reuse ratio rho_Q),
as the oracle takes them: a KV head's mask row is the union in visit order and
membership[qb, h, k] marks the entries of q head h.

Checked against: the worked example the notes print; per-head brute-force softmax
over each head's own support set (skipping off); per-head runs of the ordered
oracle on each head's own row (skipping on); the shared-mask oracle when every
head takes every entry; and, for the union builder, the shared builder at G = 1,
brute-force per-head selection and the shared builder's full candidate order."""
import json
import os

import numpy as np
import pytest

from oracle import maskref, osk

D = 128
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pageweaver_union_example.json")


def case(lens, hq, hkv, seed, structured=False):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    nb = [-(-L // 64) for L in lens]
    q = (rng.standard_normal((T, hq, D)) / np.sqrt(D)).astype(np.float32)
    k = rng.standard_normal((sum(nb), hkv, 64, D)).astype(np.float32)
    if structured:
        # a few blocks whose keys align with a shared query direction per KV head
        u = rng.standard_normal((hkv, D)).astype(np.float32)
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        for g in range(hkv):
            q[:, g * (hq // hkv):(g + 1) * (hq // hkv), :] += 0.5 * u[g]
            hot = rng.choice(sum(nb), size=max(1, sum(nb) // 4), replace=False)
            k[hot, g] += 2.0 * u[g]
    else:
        k /= np.sqrt(D)
    v = (rng.standard_normal((sum(nb), hkv, 64, D)) / np.sqrt(D)).astype(np.float32)
    pt = np.full((len(lens), max(nb)), -1, dtype=np.int32)
    perm = rng.permutation(sum(nb))
    pos = 0
    for s, n in enumerate(nb):
        pt[s, :n] = perm[pos:pos + n]
        pos += n
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, v, pt, cu, nb


def random_union(cu, nb, hq, hkv, seed, junk=True):
    """Union rows without repeated ids (random causal blocks in random order, plus
    junk entries) and a random membership with every valid entry in some head."""
    rng = np.random.default_rng(seed)
    rows = []
    for s, n in enumerate(nb):
        for i in range(n):
            rows.append((i, n))
    width = max(i + 1 for i, _ in rows) + (3 if junk else 0)
    om = np.full((len(rows), hkv, width), -1, dtype=np.int32)
    ml = np.zeros((len(rows), hkv), dtype=np.int32)
    mem = np.zeros((len(rows), hq, width), dtype=np.uint8)
    G = hq // hkv
    for qb, (i, n) in enumerate(rows):
        for g in range(hkv):
            ids = rng.permutation(i + 1)[: rng.integers(1, i + 2)].tolist()
            if junk and rng.random() < 0.5:
                ids.insert(int(rng.integers(0, len(ids) + 1)), int(rng.choice([-1, n + 3, i + 1 if i + 1 < n else -5])))
            om[qb, g, : len(ids)] = ids
            ml[qb, g] = len(ids)
            m = (rng.random((G, len(ids))) < 0.6).astype(np.uint8)
            m[rng.integers(0, G, len(ids)), np.arange(len(ids))] = 1
            mem[qb, g * G:(g + 1) * G, : len(ids)] = m
    return om, ml, mem


def head_rows(om, ml, mem, h, g):
    """Head h's own mask row: the union row's entries that belong to it."""
    nqb, _, W = om.shape
    out = np.full((nqb, 1, W), -1, dtype=np.int32)
    ln = np.zeros((nqb, 1), dtype=np.int32)
    pos = np.full((nqb, W), -1, dtype=np.int64)   # union position -> position in the head's row
    for qb in range(nqb):
        n = 0
        for kk in range(ml[qb, g]):
            if mem[qb, h, kk]:
                out[qb, 0, n] = om[qb, g, kk]
                pos[qb, kk] = n
                n += 1
        ln[qb, 0] = n
    return out, ln, pos


def test_worked_union_example():
    ex = json.load(open(GOLDEN))
    sets = [ex["sets"]["q0"], ex["sets"]["q2"]]
    u, m = maskref.union_and_membership(sets, lambda j: j)
    assert u.tolist() == ex["union"]
    assert m.tolist() == [ex["membership"]["q0"], ex["membership"]["q2"]]
    assert int(m.sum()) == ex["query_page_selections"] and len(u) == ex["pages_traversed"]
    assert maskref.reuse_ratio([len(s) for s in sets], [len(u)]) == ex["reuse_ratio"]


def test_membership_is_per_head_support_set_without_skipping():
    lens = [64 * 6 + 17, 64 * 3]
    hq, hkv = 8, 2
    q, k, v, pt, cu, nb = case(lens, hq, hkv, 5)
    om, ml, mem = random_union(cu, nb, hq, hkv, 9)
    res = osk.osk_reference(q, k, v, pt, cu, om, ml, -1.0, membership=mem)
    G = hq // hkv
    for h in range(hq):
        g = h // G
        omh, mlh, _ = head_rows(om, ml, mem, h, g)
        out, lse = osk.brute_force_attention(q[:, [h]], k[:, [g]], v[:, [g]], pt, cu, omh, mlh)
        np.testing.assert_allclose(res["out"][:, h], out[:, 0], atol=1e-12)
        np.testing.assert_allclose(res["lse"][:, h], lse[:, 0], atol=1e-12)


def test_membership_with_skipping_equals_each_heads_own_ordered_run():
    lens = [64 * 9 + 5]
    hq, hkv = 4, 1
    q, k, v, pt, cu, nb = case(lens, hq, hkv, 11, structured=True)
    om, ml, mem = random_union(cu, nb, hq, hkv, 12, junk=True)
    base = osk.osk_reference(q, k, v, pt, cu, om, ml, -1.0, membership=mem, compute_output=False)
    mg = base["margins"][np.isfinite(base["margins"])]
    tau = float(np.quantile(mg[mg < 0], 0.5)) if (mg < 0).any() else -0.1
    delta = lens[0] * np.exp(tau)
    res = osk.osk_reference(q, k, v, pt, cu, om, ml, delta, membership=mem)
    skipped = 0
    for h in range(hq):
        omh, mlh, pos = head_rows(om, ml, mem, h, 0)
        one = osk.osk_reference(q[:, [h]], k, v, pt, cu, omh, mlh, delta)
        np.testing.assert_allclose(res["out"][:, h], one["out"][:, 0], atol=1e-12)
        np.testing.assert_allclose(res["lse"][:, h], one["lse"][:, 0], atol=1e-12)
        for qb in range(om.shape[0]):
            for kk in range(om.shape[2]):
                if pos[qb, kk] >= 0:
                    assert res["decisions"][qb, h, kk] == one["decisions"][qb, 0, pos[qb, kk]]
                    skipped += int(res["decisions"][qb, h, kk] == osk.NOT_COMPUTED_SKIP)
                else:
                    assert res["decisions"][qb, h, kk] == osk.NOT_VISITED
                    assert np.isnan(res["margins"][qb, h, kk])
    assert skipped > 0


def test_full_membership_is_the_shared_mask():
    lens = [64 * 5 + 3, 100]
    hq, hkv = 8, 2
    q, k, v, pt, cu, nb = case(lens, hq, hkv, 21, structured=True)
    om, ml = maskref.build_order_mask(q, k, pt, cu, hkv, 0.5)
    ones = np.ones((om.shape[0], hq, om.shape[2]), np.uint8)
    for delta in (-1.0, float(sum(lens)) * np.exp(-0.05)):
        a = osk.osk_reference(q, k, v, pt, cu, om, ml, delta)
        b = osk.osk_reference(q, k, v, pt, cu, om, ml, delta, membership=ones)
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])


def test_union_builder_at_one_head_per_group_is_the_shared_builder():
    lens = [64 * 11 + 40, 64 * 4]
    q, k, v, pt, cu, nb = case(lens, 2, 2, 31, structured=True)
    for b1, flags in ((0.3, 3), (0.5, 1), (0.0, 3)):
        om, ml = maskref.build_order_mask(q, k, pt, cu, 2, b1, flags=flags)
        uo, ul, mem, hl = maskref.build_union_mask(q, k, pt, cu, 2, b1, flags=flags, width=om.shape[2])
        np.testing.assert_array_equal(uo, om)
        np.testing.assert_array_equal(ul, ml)
        np.testing.assert_array_equal(hl, ml)
        W = om.shape[2]
        assert np.array_equal(mem != 0, np.arange(W)[None, None, :] < ml[:, :, None])


def test_union_builder_sets_and_order():
    lens = [64 * 13 + 9]
    hq, hkv, b1 = 8, 2, 0.25
    G = hq // hkv
    q, k, v, pt, cu, nb = case(lens, hq, hkv, 41, structured=True)
    uo, ul, mem, hl = maskref.build_union_mask(q, k, pt, cu, hkv, b1)
    # every candidate in the shared builder's order (score descending, id ascending)
    full, fl = maskref.build_order_mask(q, k, pt, cu, hkv, 1.0)
    n = nb[0]
    L = lens[0]
    for i in range(n):
        rows = range(i * 64, min(L, (i + 1) * 64))
        for g in range(hkv):
            u = uo[i, g, : ul[i, g]].tolist()
            # the union keeps the shared order
            assert u == [j for j in full[i, g, : fl[i, g]].tolist() if j in set(u)]
            for hh in range(G):
                h = g * G + hh
                # brute-force selection for head h: explicit means and dot products
                qm = [sum(float(q[t, h, dd]) for t in rows) / len(rows) for dd in range(D)]
                scores = []
                for j in range(i + 1):
                    toks = range(j * 64, min(L, (j + 1) * 64))
                    km = [sum(float(k[pt[0, j], g, t - j * 64, dd]) for t in toks) / len(toks) for dd in range(D)]
                    scores.append(sum(a * b for a, b in zip(qm, km)))
                forced = [0] + ([i] if i != 0 else [])
                rest = sorted((j for j in range(i + 1) if j not in forced), key=lambda j: (-scores[j], j))
                want = set(forced) | set(rest[: maskref.keep_count(np.float32(b1), len(rest))])
                got = {u[kk] for kk in range(len(u)) if mem[i, h, kk]}
                assert got == want, (i, h)
                assert hl[i, h] == len(want)
                assert not mem[i, h, ul[i, g]:].any()


def test_identical_heads_give_the_shared_row_and_full_reuse():
    lens = [64 * 9 + 1]
    hq, hkv = 8, 2
    q, k, v, pt, cu, nb = case(lens, hq, hkv, 51, structured=True)
    G = hq // hkv
    for g in range(hkv):
        q[:, g * G:(g + 1) * G] = q[:, g * G:g * G + 1]
    om, ml = maskref.build_order_mask(q, k, pt, cu, hkv, 0.3)
    uo, ul, mem, hl = maskref.build_union_mask(q, k, pt, cu, hkv, 0.3)
    W = om.shape[2]
    np.testing.assert_array_equal(uo[:, :, :W], om)
    assert (uo[:, :, W:] == -1).all()
    np.testing.assert_array_equal(ul, ml)
    assert maskref.reuse_ratio(hl, ul) == G
