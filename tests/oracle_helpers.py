"""Small hand-built problems for the CPU pin tests (random numbers only)."""
import numpy as np


def make_problem(rng, seq_lens, Hq, Hkv, d, P, shuffled=False, scale=1.0):
    """Random q [T,Hq,d], pools [n_phys,Hkv,P,d], page table and cu_seqlens."""
    S = len(seq_lens)
    pages = [-(-L // P) for L in seq_lens]
    cu = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    n_phys = sum(pages) + (3 if shuffled else 0)
    perm = rng.permutation(n_phys) if shuffled else np.arange(n_phys)
    pt = np.full((S, max(pages)), -1, dtype=np.int64)
    off = 0
    for s in range(S):
        pt[s, : pages[s]] = perm[off: off + pages[s]]
        off += pages[s]
    T = int(cu[-1])
    q = rng.standard_normal((T, Hq, d)) * scale
    k = rng.standard_normal((n_phys, Hkv, P, d)) * scale
    v = rng.standard_normal((n_phys, Hkv, P, d))
    return q, k, v, pt, cu


def random_masks(rng, seq_lens, Hkv, P, width, junk=True, full_fraction=0.6):
    """Random ordered masks; with junk, rows also hold -1, out-of-range,
    non-causal and repeated ids that must not be visited."""
    rows = []
    for L in seq_lens:
        n = -(-L // P)
        for i in range(n):
            rows.append((i, n))
    om = np.full((len(rows), Hkv, width), -1, dtype=np.int64)
    ml = np.zeros((len(rows), Hkv), dtype=np.int64)
    for qb, (i, n) in enumerate(rows):
        for g in range(Hkv):
            cand = rng.permutation(i + 1)
            keep = cand[: max(1, int(round(full_fraction * (i + 1))))]
            row = list(keep)
            if junk:
                extra = [-1, n, n + 5, i + 1 if i + 1 < n else -7]
                if len(keep):
                    extra.append(int(keep[0]))          # a repeat
                for e in extra:
                    if rng.random() < 0.5:
                        row.insert(int(rng.integers(0, len(row) + 1)), int(e))
            row = row[:width]
            om[qb, g, : len(row)] = row
            ml[qb, g] = len(row)
    return om, ml
