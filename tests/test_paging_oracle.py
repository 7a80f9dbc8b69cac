"""Pins of the logical-block view of a KV cache paged below the block size (CoSA
Appendix D.1, "CoSA settings": b and b_p configured independently): re-paging a
64-token pool at 16 or 32 tokens per physical page under a random physical
permutation must leave every oracle result unchanged, and a block with one
unusable physical page behaves as an invalid logical id."""
import numpy as np
import pytest

from oracle import kap, maskref, osk, paging

D = 128


def case(lens, hq, hkv, seed):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    q = (rng.standard_normal((T, hq, D)) / np.sqrt(D)).astype(np.float32)
    nb = [-(-L // 64) for L in lens]
    k64 = rng.standard_normal((sum(nb), hkv, 64, D)).astype(np.float32)
    v64 = (rng.standard_normal((sum(nb), hkv, 64, D)) / np.sqrt(D)).astype(np.float32)
    pt64 = np.full((len(lens), max(nb)), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(nb):
        pt64[s, :n] = np.arange(pos, pos + n)
        pos += n
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k64, v64, pt64, cu


def repage(k64, v64, pt64, lens, bp, seed):
    """The same tokens stored at bp tokens per physical page, pages shuffled."""
    sub = 64 // bp
    n_small = k64.shape[0] * sub
    perm = np.random.default_rng(seed).permutation(n_small + 5)
    hkv = k64.shape[1]
    kp = np.zeros((n_small + 5, hkv, bp, D), np.float32)
    vp = np.zeros_like(kp)
    pt = np.full((len(lens), pt64.shape[1] * sub), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        for j in range(-(-L // 64)):
            for x in range(sub):
                if j * 64 + x * bp >= L:
                    continue
                dst = perm[pt64[s, j] * sub + x]
                kp[dst] = k64[pt64[s, j], :, x * bp:(x + 1) * bp]
                vp[dst] = v64[pt64[s, j], :, x * bp:(x + 1) * bp]
                pt[s, j * sub + x] = dst
    return kp, vp, pt


@pytest.mark.parametrize("bp", [16, 32])
def test_repaged_pool_gives_identical_results(bp):
    lens = [64 * 5 + 21, 64 * 3, 40]
    q, k64, v64, pt64, cu = case(lens, 8, 2, 3)
    kp, vp, pt = repage(k64, v64, pt64, lens, bp, 7)
    kl, vl, ptl = paging.logical_view(kp, vp, pt, cu, bp)
    om, ml = maskref.build_order_mask(q, k64, pt64, cu, 2, 0.5)
    om2, ml2 = maskref.build_order_mask(q, kl, ptl, cu, 2, 0.5)
    np.testing.assert_array_equal(om, om2)
    np.testing.assert_array_equal(ml, ml2)
    a = osk.osk_reference(q, k64, v64, pt64, cu, om, ml, delta=float(np.exp(-0.05) * max(lens)))
    b = osk.osk_reference(q, kl, vl, ptl, cu, om, ml, delta=float(np.exp(-0.05) * max(lens)))
    for key in a:
        x, y = np.asarray(a[key]), np.asarray(b[key])
        np.testing.assert_array_equal(np.isnan(x), np.isnan(y)) if x.dtype.kind == "f" else None
        np.testing.assert_array_equal(np.nan_to_num(x, nan=-3.0), np.nan_to_num(y, nan=-3.0))
    ka = kap.build_kap_mask(q, k64, pt64, cu, 2, 16, kap.MODE_TOP_P, 0.9)
    kb = kap.build_kap_mask(q, kl, ptl, cu, 2, 16, kap.MODE_TOP_P, 0.9)
    for x, y in zip(ka, kb):
        np.testing.assert_array_equal(np.nan_to_num(x, nan=-3.0), np.nan_to_num(y, nan=-3.0))


def test_unusable_physical_page_invalidates_its_block():
    lens = [64 * 4]
    q, k64, v64, pt64, cu = case(lens, 2, 1, 5)
    kp, vp, pt = repage(k64, v64, pt64, lens, 16, 2)
    pt_bad = pt.copy()
    pt_bad[0, 2 * 4 + 1] = -1                       # one of block 2's four physical pages
    kl, vl, ptl = paging.logical_view(kp, vp, pt_bad, cu, 16)
    assert ptl[0, 2] == -1 and np.all(ptl[0, [0, 1, 3]] >= 0)
    # the prefill oracle then gives block 2's page no interaction, exactly as an invalid id
    om = np.array([[[3, 2, 1, 0]]] * 4, dtype=np.int32).reshape(4, 1, 4)
    ml = np.full((4, 1), 4, dtype=np.int32)
    a = osk.osk_reference(q, kl, vl, ptl, cu, om, ml, delta=-1.0)
    pt64b = pt64.copy()
    pt64b[0, 2] = -1
    b = osk.osk_reference(q, k64, v64, pt64b, cu, om, ml, delta=-1.0)
    np.testing.assert_array_equal(np.nan_to_num(np.asarray(a["out"]), nan=-3.0), np.nan_to_num(np.asarray(b["out"]), nan=-3.0))
