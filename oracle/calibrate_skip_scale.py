"""Freeze the skip scale Delta of each workload from the fp64 oracle's margins.

TEST INFRASTRUCTURE (see oracle/osk.py).  Writes the workload parameter table
block_sparse_long_osk_amd/skip_scales.json (the package reads each workload's
Delta from it); calls only oracle/ and the seeded input generator.  Usage:  python -m oracle.calibrate_skip_scale [names...]

Why the margins suffice: Algorithm A of CoSA updates the running max before the
skip test whether or not the page is skipped, so every visit's margin
max_r(m_loc[r] - m[r]) is fixed by the logits and the visit order alone; a page
is skipped iff margin < ln(Delta / L_s), i.e. iff margin + ln L_s < ln Delta.
The skip ratio is therefore the empirical distribution of margin + ln L_s,
evaluated at ln Delta, exactly and monotonically.

Readings (the pages give the rule, not these operating points):
* workloads whose second stage names no level: Delta is set so that 40 % of the
  visited (q head, block, page) triples are skipped, then rounded to 4
  significant figures (the realized ratio is recorded);
* the i.i.d. 16K workload asks for a trim its inputs cannot reach: 91 % of its
  visits have margin exactly 0 (one of the 64 rows finds a new maximum), so
  Delta = L exp(-1e-5) skips essentially every visit whose margin is negative,
  the attainable maximum; the realized ratio is recorded next to the request.
"""
from __future__ import annotations

import json
import math
import os
import sys
import time

import numpy as np

from oracle import maskref, osk

OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "block_sparse_long_osk_amd", "skip_scales.json")
TARGET_SKIP = 0.40
IID_TAU = -1e-5


def visit_statistics(name: str):
    """x = margin + ln L_s of every visited (block, q head, page) of a workload."""
    from block_sparse_long_osk_amd import inputs      # seeded generator only
    wl = inputs.WORKLOADS[name]
    bt = inputs.generate(wl)
    q = inputs.bf16_bits_to_f32(bt.q)
    k = inputs.bf16_bits_to_f32(bt.k_pool)
    v = inputs.bf16_bits_to_f32(bt.v_pool)
    om, ml = maskref.build_order_mask(q, k, bt.page_table, bt.cu_seqlens, wl.num_kv_heads, wl.budget1)
    res = osk.osk_reference(q, k, v, bt.page_table, bt.cu_seqlens, om, ml, delta=-1.0,
                            compute_output=False)
    m = res["margins"]
    lnL = np.zeros(m.shape[0])
    for s in range(bt.num_seqs):
        lnL[bt.cu_qblocks[s]:bt.cu_qblocks[s + 1]] = math.log(wl.seq_lens[s])
    vis = np.isfinite(m)
    x = (m + lnL[:, None, None])[vis]
    return wl, x, int(ml.sum()), m[vis]


def calibrate(name: str) -> dict:
    t0 = time.time()
    wl, x, n_mask_entries, margins = visit_statistics(name)
    n = x.size
    if wl.generator == "iid":
        L = wl.seq_lens[0]
        delta = float(f"{L * math.exp(IID_TAU):.7g}")
        rule = "iid: Delta = L exp(-1e-5), the largest attainable trim"
    else:
        xs = np.sort(x)
        kq = int(round(TARGET_SKIP * n))
        theta = 0.5 * (xs[kq - 1] + xs[kq])
        delta = float(f"{math.exp(theta):.4g}")
        rule = "40 % of visited (q head, block, page) triples skipped, Delta rounded to 4 significant figures"
    ln_delta = math.log(delta)
    skipped = x < ln_delta
    near = np.abs(x - ln_delta) < osk.NEAR_TIE
    rec = {
        "delta": delta,
        "rule": rule,
        "taus": [math.log(delta / L) for L in wl.seq_lens],
        "visits_per_q_head": int(n),
        "skip_ratio": float(skipped.mean()),
        "near_tie_visits": int(near.sum()),
        "zero_margin_fraction": float((margins == 0).mean()),
        "margin_quantiles": {str(p): float(np.quantile(margins, p)) for p in (0.05, 0.1, 0.25, 0.4, 0.5)},
        "skip_ratio_at_delta_2000": float((x < math.log(2000.0)).mean()),
        "seconds": round(time.time() - t0, 1),
    }
    return rec


def main(argv):
    from block_sparse_long_osk_amd import inputs
    names = argv or [n for n in inputs.WORKLOAD_ORDER if inputs.WORKLOADS[n].skipping]
    table = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            table = json.load(f)
    table["_provenance"] = ("written by oracle/calibrate_skip_scale.py from the fp64 oracle's margins "
                            "on the seeded workloads; see that script's docstring for the readings")
    for name in names:
        rec = calibrate(name)
        print(name, json.dumps(rec), flush=True)
        table[name] = rec
        with open(OUT, "w") as f:
            json.dump(table, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
