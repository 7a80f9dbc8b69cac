"""Logical blocks (64 or 128 tokens) over a KV cache paged at another physical page size.

TEST INFRASTRUCTURE ONLY (see oracle/osk.py).

Source: CoSA Appendix D.1 ("CoSA settings"): the attention block size b and the
number of tokens b_p per stored page are two separate settings, so when they differ one logical
block maps onto several stored pages (or part of one).  The section gives no more
detail; the readings taken here are:

* logical block j of a sequence holds its tokens b j .. b j + b - 1 (b = 64 or 128);
  token t is stored in physical page page_table[t // b_p] at row t % b_p (b_p
  divides b);
* a logical block is usable only if every physical page holding one of its tokens
  t < L is a valid page (0 <= id < n_phys); otherwise it behaves as an invalid
  logical id (it adds no interaction).

logical_view() rebuilds the pool at the logical block size, with one logical page
per (sequence, block) and a logical page table (-1 for unusable blocks), so that
the oracles, which take the block as their page size, apply unchanged.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


def logical_view(k_pool, v_pool, page_table, cu_seqlens, page_size: int, block: int = BLOCK):
    """Returns (k_log, v_log, pt_log): pools [n_blocks_total, Hkv, block, d] (rows past
    a sequence's end are zero) and a page table [S, max_blocks] of logical page ids."""
    if block % page_size != 0:
        raise ValueError("the physical page size must divide the block size")
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool) if v_pool is not None else None
    n_phys, hkv, P, d = k_pool.shape
    assert P == page_size
    S = len(cu_seqlens) - 1
    lens = [int(cu_seqlens[s + 1] - cu_seqlens[s]) for s in range(S)]
    nblk = [-(-L // block) for L in lens]
    total = sum(nblk)
    max_blocks = max(nblk) if nblk else 1
    k_log = np.zeros((max(total, 1), hkv, block, d), dtype=k_pool.dtype)
    v_log = np.zeros_like(k_log) if v_pool is not None else None
    pt_log = np.full((S, max_blocks), -1, dtype=np.int32)
    pos = 0
    for s in range(S):
        L = lens[s]
        for j in range(nblk[s]):
            toks = np.arange(j * block, min(L, (j + 1) * block))
            phys = np.asarray(page_table[s])[toks // page_size]
            if np.all((phys >= 0) & (phys < n_phys)):
                k_log[pos, :, : toks.size, :] = k_pool[phys, :, toks % page_size, :].transpose(1, 0, 2)
                if v_pool is not None:
                    v_log[pos, :, : toks.size, :] = v_pool[phys, :, toks % page_size, :].transpose(1, 0, 2)
                pt_log[s, j] = pos
            pos += 1
    return k_log, v_log, pt_log
