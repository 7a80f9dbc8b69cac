"""Plain fp64 CPU oracle of ordered block-sparse prefill attention with in-kernel skipping.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the package's smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library.

What it computes (sources are the pages this project follows):

* Support set -- PageWeaver notes, section 2.1, Eq. (1)-(2): a query at causal
  position c of a sequence of valid length L attends to the tokens
  A = {t : floor(t/P) in S, 0 <= t < L, t <= c}, where S is the set of valid,
  de-duplicated logical page ids; invalid ids add no interaction, duplicates add
  no mass and an empty support gives a zero output.
* Ordered online softmax with in-kernel skip -- CoSA, section 3.1 Eq. (1)-(2),
  section 3.3 Eq. (5) and Appendix C, Algorithm A (attention loop): per query
  block i and q head, the pages of the block's computation-order mask are visited
  in mask order; for each page the exact scaled logits S give the local row max
  m_loc, the running max is updated m <- max(m, m_loc) before the test, and the
  value side (exp, row sum, output rescale and P V) is skipped when the skip
  scale Delta > 0 and max_r(m_loc[r] - m[r]) < ln(Delta / N).
* N is the sequence's valid length L (the threshold adapts to context length,
  CoSA section 3.3); the vote is taken over the block's valid rows (rows past L
  do not vote); a row that sees no key of a page does not veto.

* Per-q-head page sets under grouped-query heads -- PageWeaver notes, section 2.2:
  the heads of a KV group traverse the union U of their sets, and a membership
  mask M[h, p] = 1[p in S_h] keeps each head's softmax to its own pages.  Here the
  mask row of a KV head is the union in visit order and membership[qb, h, k] says
  whether entry k belongs to q head h; a head takes part in a visit (key side,
  running max, vote, value side) only at its own entries, so it sees exactly its
  own pages in the union's order.

Decision codes: 0 = computed, 1 = skipped in-kernel, 2 = not visited (mask
padding, an id outside [0, n_pages), a non-causal id j > i, a repeated id, a
page whose page-table entry lies outside the physical pool, or an entry outside
the head's membership).
Margins are in natural-log units of the scaled logits; NaN where not visited.

All arithmetic is float64 on the exact (bfloat16-valued) inputs.  The batched
version steps all query blocks of one (sequence, KV head) through the visit index
together; each block's own sequence of operations is exactly the algorithm's.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np

NOT_COMPUTED_SKIP = 1
COMPUTED = 0
NOT_VISITED = 2
NEAR_TIE = 1e-3  # decisions within this distance of the threshold may go either way


# ----------------------------------------------------------------------------
# support set (PageWeaver notes, section 2.1, Eq. (1))
# ----------------------------------------------------------------------------
def support_set(page_ids: Iterable[int], page_size: int, valid_len: int, causal_pos: int) -> List[int]:
    """Tokens a query attends to: pages in S (valid, distinct), t < L and t <= c."""
    n_pages = -(-valid_len // page_size)
    selected = {int(j) for j in page_ids if 0 <= int(j) < n_pages}
    return [t for t in range(valid_len) if (t // page_size) in selected and t <= causal_pos]


def softmax_attention_row(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray,
                          sm_scale: float):
    """o = sum_t exp(s_t) v_t / sum_t exp(s_t) with s_t = sm_scale q.k_t (Eq. (2));
    zero output and LSE -inf for an empty support."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1]), -math.inf
    s = sm_scale * (keys.astype(np.float64) @ q_row.astype(np.float64))
    mx = s.max()
    w = np.exp(s - mx)
    denom = w.sum()
    return (w @ values.astype(np.float64)) / denom, mx + math.log(denom)


# ----------------------------------------------------------------------------
# canonical visit list of one mask row
# ----------------------------------------------------------------------------
def usable_pages(pt_row, n_pages: int, n_phys: int) -> np.ndarray:
    """[n_pages] bool: logical page j of the sequence has a physical page in the pool.

    PageWeaver notes, section 2.1 conventions: an id that does not name a stored
    page adds no interaction.  A page-table entry outside [0, n_phys) (the -1 of an
    unmapped page, or an id past the pool) therefore makes its logical page
    unusable: a mask entry naming it is not visited.
    """
    pt = np.asarray(pt_row, dtype=np.int64).reshape(-1)
    ok = np.zeros(max(n_pages, 0), dtype=bool)
    w = min(n_pages, pt.shape[0])
    ok[:w] = (pt[:w] >= 0) & (pt[:w] < n_phys)
    return ok


def canonical_visits(row: Sequence[int], length: int, block_index: int, n_pages: int,
                     usable: Optional[np.ndarray] = None) -> List[tuple]:
    """(position k, logical page j) pairs that are visited, in mask order.

    Entries past `length`, ids outside [0, n_pages), ids after the block (j > i),
    pages without a physical page in the pool (usable[j] false) and repeats of an
    id already visited are not visited.
    """
    seen = set()
    out = []
    for k in range(min(int(length), len(row))):
        j = int(row[k])
        if j < 0 or j >= n_pages or j > block_index or j in seen:
            continue
        if usable is not None and not usable[j]:
            continue
        seen.add(j)
        out.append((k, j))
    return out


# ----------------------------------------------------------------------------
# brute force: softmax over an explicit support (tiny inputs only)
# ----------------------------------------------------------------------------
def brute_force_attention(q, k_pool, v_pool, page_table, cu_seqlens, order_mask, mask_len,
                          page_size: int = 64, sm_scale: Optional[float] = None,
                          kept_pages: Optional[Dict[tuple, Sequence[int]]] = None):
    """Per-token softmax over the support set of its block's mask row.

    kept_pages optionally maps (qblock, q_head) -> logical page ids to use instead
    of the mask row (used to express "softmax over the pages that were computed").
    Returns (out [T, Hq, d], lse [T, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    if sm_scale is None or sm_scale <= 0:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.zeros((T, Hq, d))
    lse = np.full((T, Hq), -math.inf)
    S = len(cu_seqlens) - 1
    qb0 = 0
    for s in range(S):
        t0, L = int(cu_seqlens[s]), int(cu_seqlens[s + 1] - cu_seqlens[s])
        n_pages = -(-L // page_size)
        usable = usable_pages(page_table[s], n_pages, k_pool.shape[0])
        # keys/values of the sequence in logical token order (zero on unusable pages,
        # which no query can see)
        keys = np.zeros((L, Hkv, d))
        vals = np.zeros((L, Hkv, d))
        for j in range(n_pages):
            if not usable[j]:
                continue
            ph = int(page_table[s][j])
            n = min(page_size, L - j * page_size)
            keys[j * page_size: j * page_size + n] = np.asarray(k_pool[ph, :, :n, :], np.float64).transpose(1, 0, 2)
            vals[j * page_size: j * page_size + n] = np.asarray(v_pool[ph, :, :n, :], np.float64).transpose(1, 0, 2)
        for i in range(n_pages):
            qb = qb0 + i
            for h in range(Hq):
                g = h // G
                if kept_pages is not None:
                    ids = kept_pages.get((qb, h), [])
                else:
                    ids = [j for _, j in canonical_visits(order_mask[qb, g], mask_len[qb, g], i, n_pages,
                                                          usable)]
                for r in range(page_size):
                    c = i * page_size + r
                    if c >= L:
                        break
                    A = support_set(ids, page_size, L, c)
                    o, e = softmax_attention_row(q[t0 + c, h], keys[A, g], vals[A, g], sm_scale)
                    out[t0 + c, h] = o
                    lse[t0 + c, h] = e
        qb0 += n_pages
    return out, lse


# ----------------------------------------------------------------------------
# ordered online softmax with in-kernel skip (CoSA Algorithm A, attention loop)
# ----------------------------------------------------------------------------
def skip_threshold(delta: float, seq_len: int) -> Optional[float]:
    """tau = ln(Delta / N) (CoSA Eq. (5)); None when skipping is disabled (Delta <= 0)."""
    if delta is None or delta <= 0:
        return None
    return math.log(delta / seq_len)


def osk_reference(q, k_pool, v_pool, page_table, cu_seqlens, order_mask, mask_len, delta: float,
                  page_size: int = 64, sm_scale: Optional[float] = None,
                  compute_output: bool = True, units: Optional[Sequence[tuple]] = None,
                  decision_override=None, chunk_blocks: int = 128, membership=None):
    """Run the ordered online softmax with in-kernel skipping.

    q: [T, Hq, d]; k_pool, v_pool: [n_phys, Hkv, P, d]; page_table: [S, max_pages];
    cu_seqlens: [S+1]; order_mask: [total_qblocks, Hkv, max_len]; mask_len:
    [total_qblocks, Hkv]; delta: skip scale (<= 0 disables skipping).

    units: optional list of (qblock, kv_head) pairs to evaluate (default: all).
    decision_override: optional callable (qb, heads, k, own_decision[nb?], margin) ->
        decisions to use instead of the oracle's own; see `replay_decisions`.
    compute_output=False runs only the logits / running-max / vote pass (the
        decisions do not depend on the value side, since m is updated before the
        test whether or not the page is skipped).
    membership: optional [total_qblocks, Hq, max_len] (nonzero = entry k of the KV
        head's row belongs to q head h); None = every head takes every entry.

    Returns dict with out [T,Hq,d], lse [T,Hq], decisions [total_qblocks,Hq,max_len]
    (uint8), margins (float64, NaN where not visited); rows of units that were not
    evaluated keep out=0, lse=-inf, decisions=255, margins=NaN.
    """
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    P = page_size
    if sm_scale is None or sm_scale <= 0:
        sm_scale = 1.0 / math.sqrt(d)
    S = len(cu_seqlens) - 1
    nqb_total = order_mask.shape[0]
    max_len = order_mask.shape[2]
    cu_qb = np.zeros(S + 1, dtype=np.int64)
    for s in range(S):
        L = int(cu_seqlens[s + 1] - cu_seqlens[s])
        cu_qb[s + 1] = cu_qb[s] + (-(-L // P))
    assert cu_qb[-1] == nqb_total

    out = np.zeros((T, Hq, d)) if compute_output else None
    lse = np.full((T, Hq), -math.inf)
    decisions = np.full((nqb_total, Hq, max_len), 255, dtype=np.uint8)
    margins = np.full((nqb_total, Hq, max_len), np.nan)

    # group requested units by (sequence, kv head)
    if units is None:
        todo = {(s, g): np.arange(cu_qb[s + 1] - cu_qb[s]) for s in range(S) for g in range(Hkv)}
    else:
        todo = {}
        for qb, g in units:
            s = int(np.searchsorted(cu_qb, qb, side="right") - 1)
            todo.setdefault((s, int(g)), []).append(int(qb - cu_qb[s]))
        todo = {key: np.array(sorted(set(v)), dtype=np.int64) for key, v in todo.items()}

    for (s, g), blocks in todo.items():
        t0 = int(cu_seqlens[s])
        L = int(cu_seqlens[s + 1] - cu_seqlens[s])
        if L == 0 or len(blocks) == 0:
            continue  # an empty sequence has no query blocks
        n_pages = -(-L // P)
        tau = skip_threshold(delta, L)
        heads = np.arange(g * G, (g + 1) * G)
        for c0 in range(0, len(blocks), chunk_blocks):
            blk = blocks[c0:c0 + chunk_blocks]
            res = _run_blocks(q, k_pool, v_pool, page_table[s], t0, L, n_pages, cu_qb[s], blk, g, heads,
                              order_mask, mask_len, tau, sm_scale, P, compute_output, decision_override,
                              membership)
            qbs = cu_qb[s] + blk
            decisions[qbs[:, None], heads[None, :], :] = res["decisions"]
            margins[qbs[:, None], heads[None, :], :] = res["margins"]
            rows = blk[:, None] * P + np.arange(P)[None, :]          # [nb, P]
            valid = rows < L
            tok = t0 + rows[valid]
            lse_b = res["lse"].transpose(0, 2, 1)[valid]             # [nvalid, G]
            lse[tok[:, None], heads[None, :]] = lse_b
            if compute_output:
                o_b = res["out"].transpose(0, 2, 1, 3)[valid]        # [nvalid, G, d]
                out[tok[:, None], heads[None, :], :] = o_b
    return {"out": out, "lse": lse, "decisions": decisions, "margins": margins}


def _run_blocks(q, k_pool, v_pool, pt_row, t0, L, n_pages, qb_base, blocks, g, heads,
                order_mask, mask_len, tau, sm_scale, P, compute_output, decision_override, membership=None):
    """All query blocks in `blocks` of one (sequence, KV head), stepped together
    through the visit index k.  State per (block, q head, row): m, l, o."""
    nb = len(blocks)
    G = len(heads)
    d = q.shape[2]
    max_len = order_mask.shape[2]
    qbs = qb_base + blocks
    # queries of the blocks, rows past L left at zero (they are masked anyway)
    rows = blocks[:, None] * P + np.arange(P)[None, :]                 # causal positions c [nb, P]
    row_valid = rows < L
    Qb = np.zeros((nb, G, P, d))
    tok = np.where(row_valid, t0 + rows, t0)
    Qb[:] = np.asarray(q[tok[:, :, None], heads[None, None, :]], dtype=np.float64).transpose(0, 2, 1, 3)
    Qb[~np.broadcast_to(row_valid[:, None, :], (nb, G, P))] = 0.0

    m = np.full((nb, G, P), -math.inf)
    lsum = np.zeros((nb, G, P))
    o = np.zeros((nb, G, P, d)) if compute_output else None
    decisions = np.full((nb, G, max_len), NOT_VISITED, dtype=np.uint8)
    margins = np.full((nb, G, max_len), np.nan)

    rows_ = np.arange(nb)
    usable = np.zeros(max(n_pages, 1), dtype=bool)
    usable[:n_pages] = usable_pages(pt_row, n_pages, k_pool.shape[0])
    seen = np.zeros((nb, max(n_pages, 1)), dtype=bool)
    lens = np.asarray(mask_len[qbs, g], dtype=np.int64)
    ids_all = np.asarray(order_mask[qbs, g, :], dtype=np.int64)
    key_off = np.arange(P)
    for k in range(max_len):
        ids = ids_all[:, k]
        visited = (k < lens) & (ids >= 0) & (ids < n_pages) & (ids <= blocks)
        jc = np.clip(ids, 0, max(n_pages - 1, 0))
        visited &= usable[jc]
        visited &= ~seen[rows_, jc]
        if not visited.any():
            continue
        seen[rows_[visited], jc[visited]] = True
        vb = np.nonzero(visited)[0]
        j = jc[vb]
        phys = np.asarray(pt_row, dtype=np.int64)[j]
        Kp = np.asarray(k_pool[phys, g], dtype=np.float64)             # [n, P, d]
        # scaled logits of this page (CoSA Eq. (1)); support t < L and t <= c (PageWeaver Eq. (1))
        Sv = sm_scale * np.matmul(Qb[vb], Kp[:, None, :, :].transpose(0, 1, 3, 2))  # [n, G, P, P]
        t_key = j[:, None] * P + key_off[None, :]                        # [n, P]
        c_row = rows[vb]                                                 # [n, P]
        vis = (t_key[:, None, :] < L) & (t_key[:, None, :] <= c_row[:, :, None]) & row_valid[vb][:, :, None]
        Sv = np.where(vis[:, None, :, :], Sv, -math.inf)
        m_loc = Sv.max(axis=3)                                           # [n, G, P]
        # running max updated before the skip test, whether or not the page is skipped
        m_old = m[vb]
        m_new = np.maximum(m_old, m_loc)
        diff = np.where(np.isneginf(m_loc), -math.inf, m_loc - np.where(np.isneginf(m_new), 0.0, m_new))
        margin = diff.max(axis=2)                                        # [n, G]
        # CoSA Eq. (5): skip iff Delta > 0 and max_r(m_loc - m) < ln(Delta / N)
        if tau is None:
            skip = np.zeros(margin.shape, dtype=bool)
        else:
            skip = margin < tau
        # heads whose set holds this entry (all of them without a membership mask)
        if membership is None:
            mem = np.ones(margin.shape, dtype=bool)
        else:
            mem = np.asarray(membership[qbs[vb][:, None], heads[None, :], k]) != 0
        if decision_override is not None:
            skip = decision_override(qbs[vb], heads, k, skip, margin, member=mem)
        decisions[vb, :, k] = np.where(mem, np.where(skip, NOT_COMPUTED_SKIP, COMPUTED), NOT_VISITED)
        margins[vb, :, k] = np.where(mem, margin, np.nan)
        m[vb] = np.where(mem[..., None], m_new, m_old)
        if not compute_output:
            continue
        # online softmax update of CoSA Eq. (2) for the pages that are not skipped
        comp = ~skip & mem                                               # [n, G]
        if not comp.any():
            continue
        alpha = np.where(np.isneginf(m_new), 1.0, np.exp(m_old - np.where(np.isneginf(m_new), 0.0, m_new)))
        p = np.exp(Sv - np.where(np.isneginf(m_new), 0.0, m_new)[..., None])   # exp(-inf) = 0
        Vp = np.asarray(v_pool[phys, g], dtype=np.float64)              # [n, P, d]
        pv = np.matmul(p, Vp[:, None, :, :])                             # [n, G, P, d]
        l_new = alpha * lsum[vb] + p.sum(axis=3)
        o_new = alpha[..., None] * o[vb] + pv
        cm = comp[:, :, None]
        lsum[vb] = np.where(cm, l_new, lsum[vb])
        o[vb] = np.where(cm[..., None], o_new, o[vb])

    # final normalisation O / l; zero output where nothing was accumulated
    res = {"decisions": decisions, "margins": margins}
    pos = lsum > 0
    with np.errstate(divide="ignore"):
        res["lse"] = np.where(pos, m + np.log(np.where(pos, lsum, 1.0)), -math.inf)
    if compute_output:
        res["out"] = np.where(pos[..., None], o / np.where(pos, lsum, 1.0)[..., None], 0.0)
    return res


# ----------------------------------------------------------------------------
# replay of another implementation's decisions at near-ties
# ----------------------------------------------------------------------------
class ReplayDecisions:
    """Decision override that accepts another implementation's choice only where the
    oracle's margin lies within NEAR_TIE of the threshold (both choices are then
    valid up to rounding); elsewhere the oracle's own decision stands and any
    difference is recorded as a disagreement.

    other: decisions array [total_qblocks, Hq, max_len] (codes 0/1/2).
    taus: per-query-block threshold array (tau of the block's sequence; NaN if off).
    """

    def __init__(self, other: np.ndarray, taus: np.ndarray):
        self.other = other
        self.taus = taus
        self.near_ties = 0
        self.near_tie_flips = 0
        self.disagreements = []  # (qb, head, k, own, other, margin)

    def __call__(self, qbs, heads, k, own_skip, margin, member=None):
        oth = self.other[qbs[:, None], heads[None, :], k]                # [n, G]
        tau = self.taus[qbs][:, None]
        if member is None:
            member = np.ones(margin.shape, dtype=bool)
        near = member & np.isfinite(tau) & (np.abs(margin - tau) < NEAR_TIE)
        self.near_ties += int(near.sum())
        oth_skip = oth == NOT_COMPUTED_SKIP
        valid_other = (oth == COMPUTED) | (oth == NOT_COMPUTED_SKIP)
        flip = near & valid_other & (oth_skip != own_skip)
        self.near_tie_flips += int(flip.sum())
        bad = member & (~near) & ((~valid_other) | (oth_skip != own_skip))
        for a, b in zip(*np.nonzero(bad)):
            self.disagreements.append((int(qbs[a]), int(heads[b]), int(k), int(own_skip[a, b]),
                                       int(oth[a, b]), float(margin[a, b])))
        return np.where(near & valid_other, oth_skip, own_skip)


def block_thresholds(cu_seqlens, delta: float, page_size: int = 64) -> np.ndarray:
    """tau of each query block's sequence (NaN when skipping is disabled)."""
    taus = []
    for s in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[s + 1] - cu_seqlens[s])
        if L == 0:
            continue  # no query blocks
        t = skip_threshold(delta, L)
        taus += [np.nan if t is None else t] * (-(-L // page_size))
    return np.array(taus, dtype=np.float64)


def full_causal_mask(cu_seqlens, num_kv_heads: int, page_size: int = 64):
    """Dense baseline mask: every causal page 0..i in ascending order."""
    rows = []
    for s in range(len(cu_seqlens) - 1):
        L = int(cu_seqlens[s + 1] - cu_seqlens[s])
        for i in range(-(-L // page_size)):
            rows.append(i + 1)
    nqb = len(rows)
    width = max(rows) if rows else 1
    om = np.full((nqb, num_kv_heads, width), -1, dtype=np.int32)
    ml = np.zeros((nqb, num_kv_heads), dtype=np.int32)
    for qb, n in enumerate(rows):
        om[qb, :, :n] = np.arange(n)
        ml[qb, :] = n
    return om, ml
