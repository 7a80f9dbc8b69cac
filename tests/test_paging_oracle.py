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
    # the prefill oracle then gives block 2 no interaction: the result is that of the
    # same rows with block 2 removed (a run that has no unusable page at all), and
    # every entry naming block 2 is logged as not visited
    om = np.array([[[3, 2, 1, 0]]] * 4, dtype=np.int32).reshape(4, 1, 4)
    ml = np.full((4, 1), 4, dtype=np.int32)
    om_rm = np.array([[[3, 1, 0, -1]]] * 4, dtype=np.int32).reshape(4, 1, 4)
    ml_rm = np.full((4, 1), 3, dtype=np.int32)
    delta = float(np.exp(-0.05) * lens[0])
    a = osk.osk_reference(q, kl, vl, ptl, cu, om, ml, delta=delta)
    b = osk.osk_reference(q, k64, v64, pt64, cu, om_rm, ml_rm, delta=delta)
    np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-12)
    rows_seeing_2 = [qb for qb in range(4) if qb >= 2]
    for qb in rows_seeing_2:
        assert np.all(a["decisions"][qb, :, 1] == osk.NOT_VISITED)
        assert np.all(np.isnan(a["margins"][qb, :, 1]))
        np.testing.assert_array_equal(a["decisions"][qb, :, [0, 2, 3]], b["decisions"][qb, :, [0, 1, 2]])


def test_128_token_blocks_match_brute_force_and_repaging():
    # CoSA Appendix D.1: b = 128 logical blocks over b_p = 64 (and 16) token pages.  The
    # oracle takes the block as its page size on the logical view; without skipping it
    # must equal per-token softmax over the support set, and the view must not depend
    # on how the tokens are paged.
    lens = [64 * 7 + 30, 64 * 4, 100]
    q, k64, v64, pt64, cu = case(lens, 4, 2, 19)
    kl, vl, ptl = paging.logical_view(k64, v64, pt64, cu, 64, block=128)
    assert kl.shape[2] == 128 and ptl.shape[1] == -(-max(lens) // 128)
    om, ml = osk.full_causal_mask(cu, 2, page_size=128)
    out_bf, lse_bf = osk.brute_force_attention(q, kl, vl, ptl, cu, om, ml, page_size=128)
    res = osk.osk_reference(q, kl, vl, ptl, cu, om, ml, delta=-1, page_size=128)
    np.testing.assert_allclose(res["out"], out_bf, atol=1e-12)
    np.testing.assert_allclose(res["lse"], lse_bf, atol=1e-12)
    # the same tokens in 16-token pages give the same 128-token view
    kp, vp, pt = repage(k64, v64, pt64, lens, 16, 3)
    kl2, vl2, ptl2 = paging.logical_view(kp, vp, pt, cu, 16, block=128)
    np.testing.assert_array_equal(ptl, ptl2)
    np.testing.assert_array_equal(kl, kl2)
    # with skipping, the 128-row vote: the builders and the oracle run at page_size 128
    om2, ml2 = maskref.build_order_mask(q, kl, ptl, cu, 2, 0.5, page_size=128)
    r2 = osk.osk_reference(q, kl, vl, ptl, cu, om2, ml2, delta=float(np.exp(-0.05) * max(lens)), page_size=128)
    assert np.isfinite(r2["out"]).all()
    km = kap.build_kap_mask(q, kl, ptl, cu, 2, 16, kap.MODE_FRACTION, 0.5, page_size=128)
    assert km[0].shape[0] == sum(-(-L // 128) for L in lens)
