"""Write the fp64 oracle's skip decision for every visit of the full-size workloads.

TEST INFRASTRUCTURE (see oracle/osk.py).  Writes tests/golden/decisions_<name>.npz;
calls only oracle/ and the seeded input generator.  Usage:

    python -m oracle.decision_fixture [names...]

Why one logits-only pass gives every decision: CoSA's attention loop (Appendix C,
Algorithm A) moves the running max to max(m, m_loc) before the skip test whether
or not the page is skipped, so each visit's margin max_r(m_loc[r] - m[r]) depends
on the logits and the visit order only, never on an earlier decision.  The visit
is skipped iff margin < ln(Delta / L_s) (CoSA section 3.3, Eq. (5)).

For each workload the mask is the oracle's own mean-pooled mask (oracle/maskref.py)
and Delta the workload's frozen skip scale.  Stored, over the visited (query block,
q head, mask entry) triples in C order of the [query block, q head, entry] log:

* skip:  packed bits, margin < tau;
* near:  packed bits, |margin - tau| < 1e-3 (either decision is accepted there);
* row_crc: CRC-32 of each (query block, KV head) mask row, so that a test can check
  that the mask it rebuilds with the oracle is the one these decisions belong to;
* the skip scale, the thresholds per sequence and the counts.
"""
from __future__ import annotations

import math
import os
import sys
import time
import zlib

import numpy as np

from oracle import maskref, osk, paging

GOLDEN = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden")
WORKLOADS = ["cfg2_16k_gqa", "cfg3_32k_structured", "cfg4_128k_structured", "cfg5_paged_2seq",
             "cfg4_128k_structured_b128"]


def fixture_path(name: str) -> str:
    return os.path.join(GOLDEN, f"decisions_{name}.npz")


def row_crcs(order_mask: np.ndarray, mask_len: np.ndarray) -> np.ndarray:
    """CRC-32 of the first mask_len int32 ids of every row."""
    nqb, hkv, _ = order_mask.shape
    out = np.zeros((nqb, hkv), dtype=np.uint32)
    om = np.ascontiguousarray(order_mask, dtype=np.int32)
    for qb in range(nqb):
        for g in range(hkv):
            out[qb, g] = zlib.crc32(om[qb, g, : int(mask_len[qb, g])].tobytes())
    return out


def oracle_views(batch):
    """(q, k, v, page_table, block) at the batch's logical block size, fp32 values."""
    from block_sparse_long_osk_amd import inputs      # seeded generator only
    q = inputs.bf16_bits_to_f32(batch.q)
    k = inputs.bf16_bits_to_f32(batch.k_pool)
    v = inputs.bf16_bits_to_f32(batch.v_pool)
    B, P = batch.block_size, k.shape[2]
    pt = batch.page_table
    if P != B:
        k, v, pt = paging.logical_view(k, v, pt, batch.cu_seqlens, P, block=B)
    return q, k, v, pt, B


def oracle_mask(batch, budget1: float):
    q, k, _, pt, B = oracle_views(batch)
    return maskref.build_order_mask(q, k, pt, batch.cu_seqlens, batch.k_pool.shape[1], budget1, page_size=B)


def write(name: str) -> dict:
    from block_sparse_long_osk_amd import inputs
    t0 = time.time()
    wl = inputs.WORKLOADS[name]
    bt = inputs.generate(wl)
    q, k, v, pt, B = oracle_views(bt)
    om, ml = maskref.build_order_mask(q, k, pt, bt.cu_seqlens, bt.k_pool.shape[1], wl.budget1, page_size=B)
    delta = inputs.skip_scale(name)
    res = osk.osk_reference(q, k, v, pt, bt.cu_seqlens, om, ml, delta=-1.0, page_size=B, compute_output=False)
    margins = res["margins"]
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    width = om.shape[2]
    visited = np.arange(width)[None, None, :] < np.repeat(ml, G, axis=1)[:, :, None]
    assert np.isfinite(margins[visited]).all() and np.isnan(margins[~visited]).all()
    taus = osk.block_thresholds(bt.cu_seqlens, delta, page_size=B)      # per query block
    m = margins[visited]
    tau_v = np.broadcast_to(taus[:, None, None], margins.shape)[visited]
    skip = m < tau_v
    near = np.abs(m - tau_v) < osk.NEAR_TIE
    lens = [int(L) for L in np.diff(bt.cu_seqlens)]
    np.savez_compressed(
        fixture_path(name), skip=np.packbits(skip), near=np.packbits(near), n=np.int64(skip.size),
        row_crc=row_crcs(om, ml), mask_len=ml.astype(np.int32), delta=np.float64(delta),
        taus=np.array([math.log(delta / L) for L in lens if L > 0]), block=np.int32(B))
    rec = dict(name=name, visits=int(skip.size), skipped=int(skip.sum()), near_ties=int(near.sum()),
               skip_ratio=float(skip.mean()), seconds=round(time.time() - t0, 1))
    print(rec, flush=True)
    return rec


def load(name: str) -> dict:
    """The stored fixture with its bit arrays unpacked (bool, length n)."""
    with np.load(fixture_path(name), allow_pickle=False) as z:
        n = int(z["n"])
        return dict(skip=np.unpackbits(z["skip"])[:n].astype(bool), near=np.unpackbits(z["near"])[:n].astype(bool),
                    row_crc=z["row_crc"], mask_len=z["mask_len"], delta=float(z["delta"]), taus=z["taus"],
                    block=int(z["block"]), n=n)


if __name__ == "__main__":
    for nm in (sys.argv[1:] or WORKLOADS):
        write(nm)
