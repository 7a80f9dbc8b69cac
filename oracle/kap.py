"""Plain fp64 CPU reference of the kernel-aware proxy (KAP) computation-order mask.

TEST INFRASTRUCTURE ONLY (see oracle/osk.py): only the tests, the package's smoke
check and the benchmark's CPU-baseline leg may use it; it shares no code with the
HIP library.

Source: CoSA section 4.2 ("Block ranking", Eq. (8)-(12); "Flag-grouped sorting",
Eq. (13)-(14)) and Appendix C (Figure A; Algorithm A, the pre-kernel proxy).  The
steps are taken in the pages' order:

1. stride-downsample queries and keys: Q~ = Stride(Q), K~ = Stride(K);
2. approximate scores S^ = Softmax(CausalMask(Q~ K~^T / sqrt(d))), row-wise;
3. MaxPool over the sampled keys of every key block: P[r, j] = max_{c in K_j} S^[r, c];
4. MaxNorm of every sampled query row: Pbar[r, j] = P[r, j] / max_j' P[r, j'];
5. block score s_ij = sum over the sampled rows r of query block i of Pbar[r, j] and
   HRM flag h_ij = 1[max over those rows of Pbar[r, j] = 1];
6. flag-grouped sort: the HRM group by s descending, then the rest by s descending;
7. stage-1 selection of the leading K_i entries, written as mask row i with -1 padding.

Readings of what the pages leave open (each is listed in the design notes):

* Stride(X) keeps the first token of every group of s consecutive tokens of a
  sequence: sample r is token r*s (r*s < L).  s divides the page size.  A sampled
  key on a page whose page-table entry lies outside the physical pool has no
  stored value and is taken as zero.
* The causal mask acts on sampled positions: sample c is visible to sample r iff
  c <= r (token c*s <= token r*s).
* d is the head dimension (scale 1/sqrt(d)).
* Blocks are the page-sized logical blocks (b = 64): the sampled keys of block j
  are c with c*s in [j*b, (j+1)*b), the sampled rows of block i likewise.
* A block none of whose sampled keys is visible to row r has P[r, j] = 0 (masked
  entries have probability 0).
* Grouped-query heads: one mask per KV head; s_ij sums over the G q heads of the
  group as well as over the block's sampled rows, and h_ij is 1 if any row of any
  of those heads attains its maximum in block j.
* Candidates are the causal blocks j <= i of the sequence.  Ties in s are broken
  by the smaller block id.
* Stage-1 selection: either a fixed fraction, K_i = ceil(b1 * (i + 1) - 1e-3)
  clamped to [1, i + 1] (the -1e-3 absorbs the binary rounding of b1), or Top-p:
  the smallest K_i >= 1 whose leading scores in the sorted order sum to at least
  p times the sum over all candidates.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

MODE_FRACTION = 0
MODE_TOP_P = 1


def sampled_rows(L: int, stride: int) -> np.ndarray:
    """Sample r is token r * stride of the sequence (first token of each stride group)."""
    return np.arange(0, L, stride, dtype=np.int64)


def gather_sampled_keys(k_pool, pt_row, L: int, g: int, stride: int, page_size: int) -> np.ndarray:
    """K~ of one KV head: [R, d] float64, sample c being token c * stride."""
    toks = sampled_rows(L, stride)
    pt = np.asarray(pt_row, dtype=np.int64).reshape(-1)
    idx = toks // page_size
    pages = np.where(idx < pt.shape[0], pt[np.minimum(idx, max(pt.shape[0] - 1, 0))], -1)
    stored = (pages >= 0) & (pages < k_pool.shape[0])
    ks = np.zeros((toks.size, k_pool.shape[-1]))
    # a sample on a page outside the pool has no stored key: it stays zero
    ks[stored] = np.asarray(k_pool[pages[stored], g, toks[stored] % page_size, :], dtype=np.float64)
    return ks


def block_ranking(qs: np.ndarray, ks: np.ndarray, i: int, stride: int, page_size: int,
                  sm_scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Eq. (8)-(12) for query block i of one q head (logit scale sm_scale, 1/sqrt(d) by
    default).

    qs: Q~ [R, d] and ks: K~ [R, d] of the sequence (float64).  Returns
    (s [i+1], hmax [i+1]): the block scores of Eq. (11) over this head's sampled
    rows of block i, and the maximum over those rows of Pbar (Eq. (12) tests it
    against 1).
    """
    per = page_size // stride                        # samples per block
    R, d = qs.shape
    rows = np.arange(i * per, min((i + 1) * per, R))
    if rows.size == 0:
        return np.zeros(i + 1), np.zeros(i + 1)
    ncols = min((i + 1) * per, R)                    # every key sample a row of block i may see
    if sm_scale is None or sm_scale <= 0:
        x = qs[rows] @ ks[:ncols].T / math.sqrt(d)   # Q~ K~^T / sqrt(d)
    else:
        x = (qs[rows] @ ks[:ncols].T) * sm_scale     # the caller's logit scale
    cols = np.arange(ncols)
    x = np.where(cols[None, :] <= rows[:, None], x, -np.inf)    # causal mask on samples
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    shat = e / e.sum(axis=1, keepdims=True)          # Eq. (8): row-wise softmax
    P = np.zeros((rows.size, i + 1))
    for j in range(i + 1):                           # Eq. (9): MaxPool over block j's samples
        c0, c1 = j * per, min((j + 1) * per, ncols)
        if c1 > c0:
            P[:, j] = shat[:, c0:c1].max(axis=1)
    Pbar = P / P.max(axis=1, keepdims=True)          # Eq. (10): MaxNorm per sampled row
    return Pbar.sum(axis=0), Pbar.max(axis=0)        # Eq. (11) and the quantity of Eq. (12)


def flag_grouped_order(s: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Eq. (13): HRM blocks (h = 1) by s descending, then the rest by s descending;
    equal scores by block id ascending."""
    ids = np.arange(s.size)
    return ids[np.lexsort((ids, -s, -h.astype(np.int64)))]


def keep_count(mode: int, budget: float, s_sorted: np.ndarray) -> int:
    """K_i of Eq. (14) for a row whose candidates' scores are s_sorted (sorted order)."""
    n = s_sorted.size
    if n == 0:
        return 0
    if mode == MODE_FRACTION:
        return max(1, min(n, math.ceil(float(budget) * n - 1e-3)))
    total = float(s_sorted.sum())
    csum = np.cumsum(s_sorted)
    k = int(np.searchsorted(csum, float(budget) * total, side="left")) + 1
    return max(1, min(n, k))


def mask_width(max_pages: int, mode: int, budget: float) -> int:
    if mode == MODE_TOP_P:
        return max(max_pages, 1)
    return max(1, min(max_pages, math.ceil(float(budget) * max_pages - 1e-3)))


def build_kap_mask(q, k_pool, page_table, cu_seqlens, num_kv_heads: int, stride: int, mode: int, budget: float,
                   page_size: int = 64, width: Optional[int] = None, blocks: Optional[List[int]] = None,
                   return_hmax: bool = False, sm_scale: Optional[float] = None):
    """KAP mask of every (query block, KV head), or of the global query blocks listed.

    Returns order_mask [nqb, Hkv, width] int32 (-1 padded), mask_len [nqb, Hkv],
    scores [nqb, Hkv, max_pages] float64 (NaN past the causal candidates) and
    flags [nqb, Hkv, max_pages] uint8 (0 past them); with `blocks`, nqb = len(blocks)
    in that order.  With return_hmax, also the largest Pbar of each (block, key block)
    over the group's sampled rows (the quantity Eq. (12) compares with 1; NaN past the
    candidates).
    """
    if page_size % stride != 0:
        raise ValueError("the stride must divide the page size")
    budget = float(np.float32(budget))               # the library takes it as fp32
    T, Hq, d = q.shape
    G = Hq // num_kv_heads
    S = len(cu_seqlens) - 1
    lens = [int(cu_seqlens[x + 1] - cu_seqlens[x]) for x in range(S)]
    pages = [-(-L // page_size) for L in lens]
    max_pages = max(pages) if pages else 1
    if width is None:
        width = mask_width(max_pages, mode, budget)
    starts = np.cumsum([0] + pages)
    want = list(range(int(starts[-1]))) if blocks is None else list(blocks)
    nqb = len(want)
    om = np.full((nqb, num_kv_heads, width), -1, dtype=np.int32)
    ml = np.zeros((nqb, num_kv_heads), dtype=np.int32)
    sc = np.full((nqb, num_kv_heads, max_pages), np.nan)
    fl = np.zeros((nqb, num_kv_heads, max_pages), dtype=np.uint8)
    hm = np.full((nqb, num_kv_heads, max_pages), np.nan)
    by_seq = {}
    for pos, qb in enumerate(want):
        sidx = int(np.searchsorted(starts, qb, side="right") - 1)
        by_seq.setdefault(sidx, []).append((pos, qb - int(starts[sidx])))
    for sidx, items in by_seq.items():
        t0, L = int(cu_seqlens[sidx]), lens[sidx]
        toks = t0 + sampled_rows(L, stride)
        for g in range(num_kv_heads):
            ks = gather_sampled_keys(k_pool, page_table[sidx], L, g, stride, page_size)
            qh = [np.asarray(q[toks, g * G + hh, :], dtype=np.float64) for hh in range(G)]
            for pos, i in items:
                s_row = np.zeros(i + 1)
                hmax = np.zeros(i + 1)
                for hh in range(G):
                    s_h, m_h = block_ranking(qh[hh], ks, i, stride, page_size, sm_scale)
                    s_row += s_h
                    hmax = np.maximum(hmax, m_h)
                h_row = (hmax == 1.0)
                order = flag_grouped_order(s_row, h_row)
                k = keep_count(mode, budget, s_row[order])
                if k > width:
                    raise ValueError(f"row needs {k} entries, mask width is {width}")
                om[pos, g, :k] = order[:k]
                ml[pos, g] = k
                sc[pos, g, : i + 1] = s_row
                fl[pos, g, : i + 1] = h_row
                hm[pos, g, : i + 1] = hmax
    if return_hmax:
        return om, ml, sc, fl, hm
    return om, ml, sc, fl
