"""Plain fp64 CPU reference of the mean-pooled-proxy computation-order mask.

TEST INFRASTRUCTURE ONLY (see oracle/osk.py).

Sources: CoSA section 4.2 Eq. (14) gives the mask format (row i lists the kept
logical page ids in visit order, -1 padding after them); the rewrite page of the
CoSA paper (section 4.2, "Implementation") describes the proxy as the dot product
of mean-pooled query-block and key-block representations, with the kept pages
visited in descending proxy order.  The pages leave the details open; the
readings taken here are:

* qbar_{g,i} = sum over the q heads h of KV group g of the mean of q_h over the
  valid rows of query block i (grouped-query heads share one page set per KV
  head, as PageWeaver notes section 2 state);
* kbar_{g,j} = mean of k_g over the tokens t < L of logical page j; a page whose
  page-table entry lies outside the physical pool has no stored keys and pools to
  zero (it scores 0 and may be kept; the prefill then does not visit it);
* score_{g,i,j} = qbar_{g,i} . kbar_{g,j} for causal pages j <= i;
* forced pages F_i = {0, i} (either can be switched off); the rest R_i are the
  other causal pages; n_keep = ceil(b1 |R_i| - 1e-3) clamped to [0, |R_i|] (the
  1e-3 absorbs the binary rounding of b1, e.g. 0.1 * 30);
* kept = F_i plus the top n_keep of R_i by (score descending, id ascending),
  all visited in (score descending, id ascending) order.

Per-q-head page sets (PageWeaver notes, section 2.2, the union U_G with membership
mask M and the logical page reuse ratio rho_Q of Eq. (3)), as build_union_mask
takes them:

* every q head h selects its own set S_h with the rule above, from its own score
  qbar_{h,i} . kbar_{g,j} (qbar_{h,i}: mean of q_h over the block's valid rows);
* the KV head's row is the union of its q heads' sets, visited in the order of
  the group's shared mask (group score descending, id ascending): each head then
  visits its own pages in that order;
* membership[qb, h, k] = 1 iff entry k of the row is in S_h;
* rho_Q = sum over heads and rows of |S_h| / sum over rows of |U|.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

FORCE_FIRST = 1
FORCE_DIAG = 2


def keep_count(budget1: float, n_rest: int) -> int:
    """n_keep = ceil(b1 * |R| - 1e-3), clamped to [0, |R|]."""
    if n_rest <= 0:
        return 0
    n = math.ceil(float(budget1) * n_rest - 1e-3)
    return max(0, min(n_rest, n))


def forced_pages(i: int, flags: int):
    f = []
    if flags & FORCE_FIRST:
        f.append(0)
    if (flags & FORCE_DIAG) and i not in f:
        f.append(i)
    return f


def row_length(i: int, budget1: float, flags: int) -> int:
    nf = len(forced_pages(i, flags))
    return nf + keep_count(budget1, i + 1 - nf)


def mask_width(max_pages: int, budget1: float, flags: int = FORCE_FIRST | FORCE_DIAG) -> int:
    """Longest row any query block of a sequence with max_pages pages can have."""
    return max((row_length(i, budget1, flags) for i in range(max(max_pages, 1))), default=1)


def pooled_proxies(q, k_pool, page_table, cu_seqlens, num_kv_heads: int, page_size: int = 64,
                   chunk_blocks: int = 256):
    """Per sequence: (qbar [n_pages, Hkv, d], kbar [n_pages, Hkv, d]) in float64."""
    T, Hq, d = q.shape
    G = Hq // num_kv_heads
    P = page_size
    out = []
    for s in range(len(cu_seqlens) - 1):
        t0, L = int(cu_seqlens[s]), int(cu_seqlens[s + 1] - cu_seqlens[s])
        n = -(-L // P)
        qbar = np.zeros((n, num_kv_heads, d))
        kbar = np.zeros((n, num_kv_heads, d))
        for i0 in range(0, n, chunk_blocks):
            i1 = min(n, i0 + chunk_blocks)
            for i in range(i0, i1):
                a, b = t0 + i * P, t0 + min(L, (i + 1) * P)
                blk = np.asarray(q[a:b], dtype=np.float64)                 # [rows, Hq, d]
                mean_h = blk.sum(axis=0) / (b - a)                         # [Hq, d]
                qbar[i] = mean_h.reshape(num_kv_heads, G, d).sum(axis=1)
                ph = int(page_table[s][i]) if i < len(page_table[s]) else -1
                cnt = min(P, L - i * P)
                if 0 <= ph < k_pool.shape[0]:
                    kbar[i] = np.asarray(k_pool[ph, :, :cnt, :], dtype=np.float64).sum(axis=1) / cnt
                # else: no stored keys, the pooled key stays zero (the block scores 0)
        out.append((qbar, kbar))
    return out


def build_order_mask(q, k_pool, page_table, cu_seqlens, num_kv_heads: int, budget1: float,
                     page_size: int = 64, flags: int = FORCE_FIRST | FORCE_DIAG,
                     width: Optional[int] = None, return_scores: bool = False):
    """Computation-order mask of every (query block, KV head).

    Returns order_mask [total_qblocks, Hkv, width] int32 (-1 padded), mask_len
    [total_qblocks, Hkv] int32 and, if asked, the scores [total_qblocks, Hkv,
    max_pages] (NaN for non-causal pages).
    """
    b1 = float(np.float32(budget1))       # the library takes the budget as fp32
    P = page_size
    S = len(cu_seqlens) - 1
    lens = [int(cu_seqlens[s + 1] - cu_seqlens[s]) for s in range(S)]
    pages = [-(-L // P) for L in lens]
    max_pages = max(pages) if pages else 1
    need = mask_width(max_pages, b1, flags)
    if width is None:
        width = need
    if width < need:
        raise ValueError(f"mask width {width} < required {need}")
    nqb = sum(pages)
    om = np.full((nqb, num_kv_heads, width), -1, dtype=np.int32)
    ml = np.zeros((nqb, num_kv_heads), dtype=np.int32)
    sc = np.full((nqb, num_kv_heads, max_pages), np.nan) if return_scores else None
    prox = pooled_proxies(q, k_pool, page_table, cu_seqlens, num_kv_heads, P)
    qb0 = 0
    for s in range(S):
        qbar, kbar = prox[s]
        n = pages[s]
        for g in range(num_kv_heads):
            scores = qbar[:, g, :] @ kbar[:, g, :].T                       # [n, n]
            for i in range(n):
                cand = np.arange(i + 1)
                srow = scores[i, : i + 1]
                if sc is not None:
                    sc[qb0 + i, g, : i + 1] = srow
                forced = forced_pages(i, flags)
                rest = np.array([j for j in cand if j not in forced], dtype=np.int64)
                nk = keep_count(b1, len(rest))
                if nk:
                    order = np.lexsort((rest, -srow[rest]))               # score desc, id asc
                    chosen = rest[order[:nk]]
                else:
                    chosen = np.zeros(0, dtype=np.int64)
                kept = np.concatenate([np.array(forced, dtype=np.int64), chosen])
                order = np.lexsort((kept, -srow[kept]))
                row = kept[order]
                om[qb0 + i, g, : len(row)] = row
                ml[qb0 + i, g] = len(row)
        qb0 += n
    if return_scores:
        return om, ml, sc
    return om, ml


# ----------------------------------------------------------------------------
# per-q-head sets, their union and membership (PageWeaver notes, section 2.2)
# ----------------------------------------------------------------------------
def union_and_membership(sets, order_key):
    """Union of the heads' sets in order_key order (ascending key; ties by id), and
    membership [n_heads, |U|] uint8 with M[h, k] = 1 iff U[k] is in sets[h]."""
    as_sets = [set(int(x) for x in s) for s in sets]
    u = sorted(set().union(*as_sets), key=lambda j: (order_key(j), j))
    mem = np.array([[1 if j in hs else 0 for j in u] for hs in as_sets], dtype=np.uint8)
    return np.array(u, dtype=np.int64), mem.reshape(len(sets), len(u))


def reuse_ratio(head_len, mask_len) -> float:
    """rho_Q (PageWeaver notes, Eq. (3)): sum_i |S_i| / sum_G |U_G|; here the sum of the
    heads' set sizes over the sum of the union row lengths."""
    den = float(np.sum(np.asarray(mask_len, dtype=np.float64)))
    return float(np.sum(np.asarray(head_len, dtype=np.float64))) / den if den > 0 else 0.0


def union_mask_width(max_pages: int, group: int, budget1: float, flags: int = FORCE_FIRST | FORCE_DIAG) -> int:
    """Longest union row: min(i + 1, G x each head's row length) over the blocks."""
    return max((min(i + 1, group * row_length(i, budget1, flags)) for i in range(max(max_pages, 1))), default=1)


def build_union_mask(q, k_pool, page_table, cu_seqlens, num_kv_heads: int, budget1: float,
                     page_size: int = 64, flags: int = FORCE_FIRST | FORCE_DIAG,
                     width: Optional[int] = None):
    """Per-q-head page sets as one union row per (query block, KV head) plus membership.

    Returns order_mask [nqb, Hkv, width] int32 (-1 padded), mask_len [nqb, Hkv] int32
    (union sizes), membership [nqb, Hq, width] uint8 and head_len [nqb, Hq] int32
    (each head's set size).
    """
    b1 = float(np.float32(budget1))
    P = page_size
    T, Hq, d = q.shape
    G = Hq // num_kv_heads
    S = len(cu_seqlens) - 1
    lens = [int(cu_seqlens[s + 1] - cu_seqlens[s]) for s in range(S)]
    pages = [-(-L // P) for L in lens]
    need = union_mask_width(max(pages) if pages else 1, G, b1, flags)
    if width is None:
        width = need
    if width < need:
        raise ValueError(f"mask width {width} < required {need}")
    nqb = sum(pages)
    om = np.full((nqb, num_kv_heads, width), -1, dtype=np.int32)
    ml = np.zeros((nqb, num_kv_heads), dtype=np.int32)
    mem = np.zeros((nqb, Hq, width), dtype=np.uint8)
    hl = np.zeros((nqb, Hq), dtype=np.int32)
    prox = pooled_proxies(q, k_pool, page_table, cu_seqlens, num_kv_heads, P)
    qb0 = 0
    for s in range(S):
        t0, L, n = int(cu_seqlens[s]), lens[s], pages[s]
        qbar, kbar = prox[s]
        # each head's own block means [n, Hq, d]
        qmean = np.zeros((n, Hq, d))
        for i in range(n):
            a, b = t0 + i * P, t0 + min(L, (i + 1) * P)
            qmean[i] = np.asarray(q[a:b], dtype=np.float64).sum(axis=0) / (b - a)
        for g in range(num_kv_heads):
            group_scores = qbar[:, g, :] @ kbar[:, g, :].T                       # [n, n], as the shared mask
            head_scores = [qmean[:, g * G + hh, :] @ kbar[:, g, :].T for hh in range(G)]
            for i in range(n):
                forced = forced_pages(i, flags)
                rest = np.array([j for j in range(i + 1) if j not in forced], dtype=np.int64)
                nk = keep_count(b1, len(rest))
                sets = []
                for hh in range(G):
                    srow = head_scores[hh][i]
                    chosen = rest[np.lexsort((rest, -srow[rest]))[:nk]] if nk else np.zeros(0, np.int64)
                    sets.append(list(forced) + chosen.tolist())
                grow = group_scores[i]
                u, m = union_and_membership(sets, lambda j: -grow[j])
                om[qb0 + i, g, : len(u)] = u
                ml[qb0 + i, g] = len(u)
                mem[qb0 + i, g * G:(g + 1) * G, : len(u)] = m
                hl[qb0 + i, g * G:(g + 1) * G] = [len(x) for x in sets]
        qb0 += n
    return om, ml, mem, hl
