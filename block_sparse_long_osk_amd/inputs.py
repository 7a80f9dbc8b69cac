"""Seeded synthetic inputs for block-sparse paged prefill attention.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic, the proxy scoring or the skip rule.  Both the HIP path and
the CPU oracle receive exactly what it produces.

Conventions
-----------
* Random streams come from ``numpy.random.default_rng([seed, stream])`` with
  stream 0 = queries, 1 = keys, 2 = values, 3 = structure, 4 = pool permutation.
* Values are drawn in fp32 and rounded to bfloat16 with round-to-nearest-even;
  the bfloat16 bit patterns (``uint16``) are the canonical inputs.
* Layouts: Q is ``[T, Hq, d]`` (sequences packed along T); the K and V pools are
  ``[n_phys, Hkv, P, d]`` pages of P = 64 tokens (or the workload's page size:
  the same tokens re-paged); page tables are ``[num_seqs, max_pages]`` int32
  padded with -1.  ``cu_qblocks`` counts the workload's logical blocks (64 or
  128 tokens).

Workloads (the five shapes the method is measured on)
----------------------------------------------------
``iid``        q, k, v ~ N(0, 1)/sqrt(d) independently.
``structured`` per KV head g: a unit query direction u_g shared by the group's
               q heads (q = z/sqrt(d) + u_g); bulk keys N(0, I); the first page
               (attention sink) and 8 planted salient pages get keys + 3 u_g;
               every page p has a unit vector w_{g,p} added 3x to its keys, and
               the queries of block i carry w_{g,i-3..i} (a 4-page local
               window); values N(0, 1)/sqrt(d).
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Dict, List, Optional

import numpy as np

PAGE = 64
HEAD_DIM = 128

STREAM_Q, STREAM_K, STREAM_V, STREAM_STRUCT, STREAM_POOL = 0, 1, 2, 3, 4


# ----------------------------------------------------------------------------
# bfloat16 helpers (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round fp32 -> bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, chunk):
        u = flat[s:s + chunk].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[s:s + chunk] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    seq_lens: tuple
    num_q_heads: int
    num_kv_heads: int
    generator: str            # "iid" | "structured"
    seeds: tuple              # one per sequence
    budget1: float            # first-stage page budget of the mean-pooled proxy mask
    pool: str = "identity"    # "identity" | "shuffled"
    pool_seed: Optional[int] = None
    pool_pages: Optional[int] = None
    skipping: bool = True     # False: skip scale fixed at -1 (disabled)
    page_size: int = 64       # tokens per physical KV page (16, 32 or 128: the same tokens re-paged)
    tokens_of: Optional[str] = None  # workload whose tokens these are (re-paged): its skip scale applies
    block_size: int = 64      # tokens per logical block (query block, mask id, vote): 64 or 128

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))


WORKLOADS: Dict[str, Workload] = {
    "cfg1_2k_mha": Workload(
        "cfg1_2k_mha", "1 head, L=2048, iid, identity pages, 50% proxy budget, skipping off",
        (2048,), 1, 1, "iid", (1001,), 0.5, skipping=False),
    "cfg2_16k_gqa": Workload(
        "cfg2_16k_gqa", "GQA 32/8, L=16384, iid, identity pages, 25% proxy budget, skipping on",
        (16384,), 32, 8, "iid", (1002,), 0.25),
    "cfg3_32k_structured": Workload(
        "cfg3_32k_structured", "GQA 32/8, L=32768, structured keys, 20% proxy budget, skipping on",
        (32768,), 32, 8, "structured", (1003,), 0.20),
    "cfg4_128k_structured": Workload(
        "cfg4_128k_structured", "GQA 32/8, L=131072, structured keys, 10% proxy budget, skipping on",
        (131072,), 32, 8, "structured", (1004,), 0.10),
    "cfg5_paged_2seq": Workload(
        "cfg5_paged_2seq", "GQA 32/8, 2 sequences L=131072+65536 in a shuffled 3072-page pool, "
        "structured keys, 10% proxy budget, skipping on",
        (131072, 65536), 32, 8, "structured", (1005, 1006), 0.10,
        pool="shuffled", pool_seed=1007, pool_pages=3072),
}
# The 128K workload with its KV cache in 16-token physical pages (four per logical block),
# shuffled: the same tokens, a different storage layout.
WORKLOADS["cfg4_128k_structured_p16"] = dataclasses.replace(
    WORKLOADS["cfg4_128k_structured"], name="cfg4_128k_structured_p16",
    description="cfg4_128k_structured with its KV cache in shuffled 16-token physical pages",
    page_size=16, pool_seed=1008, tokens_of="cfg4_128k_structured")
# The 128K workload under 128-token logical blocks (one skip vote per 128-row query
# block) over its 64-token physical pages: two pages per block.
WORKLOADS["cfg4_128k_structured_b128"] = dataclasses.replace(
    WORKLOADS["cfg4_128k_structured"], name="cfg4_128k_structured_b128",
    description="cfg4_128k_structured with 128-token logical blocks over 64-token pages",
    block_size=128, tokens_of="cfg4_128k_structured")
WORKLOAD_ORDER = ["cfg1_2k_mha", "cfg2_16k_gqa", "cfg3_32k_structured",
                  "cfg4_128k_structured", "cfg5_paged_2seq"]


def small_workload(name: str, seq_lens, num_q_heads: int, num_kv_heads: int,
                   generator: str = "iid", seed: int = 7, budget1: float = 0.5,
                   pool: str = "identity") -> Workload:
    """A reduced-size workload with the same recipe (for parity tests)."""
    seeds = tuple(seed + 17 * s for s in range(len(seq_lens)))
    n_pages = sum(-(-L // PAGE) for L in seq_lens)
    return Workload(name, "reduced", tuple(int(L) for L in seq_lens), num_q_heads, num_kv_heads,
                    generator, seeds, budget1, pool=pool,
                    pool_seed=seed + 5 if pool == "shuffled" else None,
                    pool_pages=(n_pages + 3) if pool == "shuffled" else None)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Batch:
    workload: Workload
    q: np.ndarray            # uint16 bf16 bits [T, Hq, d]
    k_pool: np.ndarray       # uint16 bf16 bits [n_phys, Hkv, P, d]
    v_pool: np.ndarray       # uint16 bf16 bits [n_phys, Hkv, P, d]
    page_table: np.ndarray   # int32 [S, max_pages] (-1 pad)
    cu_seqlens: np.ndarray   # int32 [S+1]
    cu_qblocks: np.ndarray   # int32 [S+1]
    salient_pages: List[np.ndarray]  # per sequence [Hkv, n_salient] (structured only)

    @property
    def num_seqs(self) -> int:
        return len(self.workload.seq_lens)

    @property
    def total_qblocks(self) -> int:
        return int(self.cu_qblocks[-1])

    @property
    def max_pages(self) -> int:
        """Page-table row length (physical pages per sequence)."""
        return int(self.page_table.shape[1])

    @property
    def block_size(self) -> int:
        return int(self.workload.block_size)

    @property
    def max_blocks(self) -> int:
        """Logical blocks a page-table row addresses."""
        return -(-self.max_pages * int(self.k_pool.shape[2]) // self.block_size)


def _unit_rows(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    x = rng.standard_normal((n, d))
    return (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)


def _gen_sequence(wl: Workload, seed: int, L: int):
    """Returns (q [L,Hq,d] f32, k [L,Hkv,d] f32, v [L,Hkv,d] f32, salient [Hkv, n])."""
    Hq, Hkv, d = wl.num_q_heads, wl.num_kv_heads, HEAD_DIM
    G = Hq // Hkv
    inv = np.float32(1.0 / math.sqrt(d))
    rq = np.random.default_rng([seed, STREAM_Q])
    rk = np.random.default_rng([seed, STREAM_K])
    rv = np.random.default_rng([seed, STREAM_V])
    q = rq.standard_normal((L, Hq, d), dtype=np.float32)
    q *= inv
    k = rk.standard_normal((L, Hkv, d), dtype=np.float32)
    v = rv.standard_normal((L, Hkv, d), dtype=np.float32)
    v *= inv
    n_pages = -(-L // PAGE)
    salient = np.zeros((Hkv, 0), dtype=np.int64)
    if L == 0:  # an empty sequence: nothing to draw structure for
        if wl.generator not in ("iid", "structured"):
            raise ValueError(wl.generator)
        return q, k, v, salient
    if wl.generator == "iid":
        k *= inv
    elif wl.generator == "structured":
        rs = np.random.default_rng([seed, STREAM_STRUCT])
        u = _unit_rows(rs, Hkv, d)                                   # [Hkv, d]
        n_sal = min(8, max(n_pages - 1, 0))
        salient = np.stack([np.sort(rs.choice(np.arange(1, n_pages), size=n_sal, replace=False))
                            if n_sal > 0 else np.zeros(0, np.int64) for _ in range(Hkv)])
        w = np.stack([_unit_rows(rs, n_pages, d) for _ in range(Hkv)])  # [Hkv, n_pages, d]
        # keys: sink + salient pages aligned with u_g, every page carries its own w_{g,p}
        for g in range(Hkv):
            marked = np.zeros(n_pages, dtype=bool)
            marked[0] = True
            marked[salient[g]] = True
            page_of_tok = np.arange(L) // PAGE
            k[:, g, :] += 3.0 * w[g][page_of_tok]
            k[marked[page_of_tok], g, :] += 3.0 * u[g]
        # queries: shared direction plus the window vectors of pages i-3..i
        wsum = np.zeros((Hkv, n_pages, d), dtype=np.float32)
        for delta in range(4):
            wsum[:, delta:, :] += w[:, :n_pages - delta, :]
        add = u[:, None, :] + wsum                                    # [Hkv, n_pages, d]
        for i0 in range(0, n_pages, 256):
            i1 = min(n_pages, i0 + 256)
            t0, t1 = i0 * PAGE, min(L, i1 * PAGE)
            blk = np.repeat(add[:, i0:i1, :], PAGE, axis=1)[:, : t1 - t0, :]   # [Hkv, t, d]
            qv = q[t0:t1].reshape(t1 - t0, Hkv, G, d)
            qv += blk.transpose(1, 0, 2)[:, :, None, :]
    else:
        raise ValueError(wl.generator)
    return q, k, v, salient


def generate(wl: Workload) -> Batch:
    """Draw the full input batch of a workload (deterministic in its seeds)."""
    Hq, Hkv, d = wl.num_q_heads, wl.num_kv_heads, HEAD_DIM
    if Hq % Hkv != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    S = len(wl.seq_lens)
    lens = np.array(wl.seq_lens, dtype=np.int64)
    pages = -(-lens // PAGE)
    cu_seqlens = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_qblocks = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    total_pages = int(pages.sum())
    max_pages = int(pages.max()) if S else 0

    if wl.pool == "identity":
        n_phys = total_pages
        phys_of = [np.arange(cu_qblocks[s], cu_qblocks[s + 1]) for s in range(S)]
    elif wl.pool == "shuffled":
        n_phys = int(wl.pool_pages)
        if n_phys < total_pages:
            raise ValueError("pool too small")
        perm = np.random.default_rng([wl.pool_seed, STREAM_POOL]).permutation(n_phys)
        phys_of = [perm[cu_qblocks[s]:cu_qblocks[s + 1]] for s in range(S)]
    else:
        raise ValueError(wl.pool)

    page_table = np.full((S, max_pages), -1, dtype=np.int32)
    for s in range(S):
        page_table[s, : pages[s]] = phys_of[s]

    T = int(cu_seqlens[-1])
    q_bits = np.empty((T, Hq, d), dtype=np.uint16)
    k_bits = np.zeros((n_phys, Hkv, PAGE, d), dtype=np.uint16)
    v_bits = np.zeros((n_phys, Hkv, PAGE, d), dtype=np.uint16)
    salient_all = []
    for s in range(S):
        L = int(lens[s])
        q, k, v, sal = _gen_sequence(wl, int(wl.seeds[s]), L)
        salient_all.append(sal)
        q_bits[cu_seqlens[s]:cu_seqlens[s + 1]] = f32_to_bf16_bits(q)
        del q
        kb = f32_to_bf16_bits(k)
        vb = f32_to_bf16_bits(v)
        del k, v
        n_full = L // PAGE
        ph = phys_of[s]
        if n_full:
            k_bits[ph[:n_full]] = kb[: n_full * PAGE].reshape(n_full, PAGE, Hkv, d).transpose(0, 2, 1, 3)
            v_bits[ph[:n_full]] = vb[: n_full * PAGE].reshape(n_full, PAGE, Hkv, d).transpose(0, 2, 1, 3)
        rem = L - n_full * PAGE
        if rem:
            k_bits[ph[n_full], :, :rem, :] = kb[n_full * PAGE:].transpose(1, 0, 2)
            v_bits[ph[n_full], :, :rem, :] = vb[n_full * PAGE:].transpose(1, 0, 2)
    if wl.block_size != PAGE:
        if wl.block_size % wl.page_size != 0:
            raise ValueError("the page size must divide the block size")
        cu_qblocks = np.concatenate([[0], np.cumsum(-(-lens // wl.block_size))]).astype(np.int32)
    bt = Batch(wl, q_bits, k_bits, v_bits, page_table, cu_seqlens, cu_qblocks, salient_all)
    if wl.page_size != PAGE:
        bt = repage(bt, wl.page_size, wl.pool_seed if wl.pool_seed is not None else 0)
    return bt


def repage(batch: Batch, page_size: int, seed: int) -> Batch:
    """The same token rows stored in a pool of page_size-token physical pages (16, 32 or
    128, from a pool of 64-token pages; a storage layout change only): the page-sized
    token ranges of every sequence go to physical pages in the order of a permutation
    drawn from (seed, stream 4), with 3 spare pages; page-table rows are -1 padded;
    rows of a page past its sequence's end are zero."""
    if batch.k_pool.shape[2] != PAGE or page_size not in (16, 32, 128):
        raise ValueError("re-pages a pool of 64-token pages into 16, 32 or 128-token pages")
    S = batch.num_seqs
    lens = np.diff(batch.cu_seqlens.astype(np.int64))
    n_new = [int(-(-L // page_size)) for L in lens]
    total = sum(n_new)
    perm = np.random.default_rng([seed, STREAM_POOL]).permutation(total + 3)
    hkv, d = batch.k_pool.shape[1], batch.k_pool.shape[3]
    k_new = np.zeros((total + 3, hkv, page_size, d), dtype=batch.k_pool.dtype)
    v_new = np.zeros_like(k_new)
    width = -(-batch.page_table.shape[1] * PAGE // page_size)
    pt = np.full((S, width), -1, dtype=np.int32)
    pos = 0
    for s in range(S):
        L = int(lens[s])
        for p in range(n_new[s]):
            dst = perm[pos]
            # token rows p*page_size .. min(L, (p+1)*page_size), taken 64-token page by page
            t = p * page_size
            t_end = min(L, (p + 1) * page_size)
            while t < t_end:
                src = batch.page_table[s, t // PAGE]
                r = t % PAGE
                n = min(PAGE - r, t_end - t)
                k_new[dst, :, t - p * page_size:t - p * page_size + n] = batch.k_pool[src, :, r:r + n]
                v_new[dst, :, t - p * page_size:t - p * page_size + n] = batch.v_pool[src, :, r:r + n]
                t += n
            pt[s, p] = dst
            pos += 1
    return dataclasses.replace(batch, k_pool=k_new, v_pool=v_new, page_table=pt)


# ----------------------------------------------------------------------------
# calibrated skip scales (written by the oracle's calibration script)
# ----------------------------------------------------------------------------
_DELTA_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "skip_scales.json")


def skip_scale(name: str) -> float:
    """Skip scale Delta of a named workload (-1 when its skipping is off)."""
    wl = WORKLOADS[name]
    if not wl.skipping:
        return -1.0
    with open(_DELTA_FILE) as f:
        table = json.load(f)
    return float(table[wl.tokens_of or name]["delta"])
