"""Device-side plumbing around the C ABI: upload a seeded batch, allocate outputs,
call the library.  torch provides device memory and streams; all computation
happens in libcosa_osk.so."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import binding
from .binding import COSA_FORCE_DIAG, COSA_FORCE_FIRST


@dataclasses.dataclass
class DeviceBatch:
    q: "torch.Tensor"            # bf16 [T, Hq, 128]
    k_pool: "torch.Tensor"       # bf16 [n_phys, Hkv, page_size, 128]
    v_pool: "torch.Tensor"
    page_table: "torch.Tensor"   # int32 [S, physical pages per sequence]
    cu_seqlens: "torch.Tensor"   # int32 [S+1]
    cu_qblocks: "torch.Tensor"   # int32 [S+1]
    total_qblocks: int
    seq_lens: tuple
    block_size: int = 64         # tokens per logical block (64 or 128)

    @property
    def num_kv_heads(self) -> int:
        return self.k_pool.shape[1]

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def max_blocks(self) -> int:
        """Logical blocks a page-table row addresses (mask ids, score rows)."""
        return -(-self.page_table.shape[1] * self.k_pool.shape[2] // self.block_size)

    def dims(self, max_mask_len: int, sm_scale: float = 0.0) -> binding.CosaOskDims:
        """Dims of the batch with rows of max_mask_len entries; sm_scale <= 0 selects 1/sqrt(128)."""
        return binding.make_dims(self.q, self.k_pool, self.page_table, self.total_qblocks, max_mask_len,
                                 sm_scale=sm_scale, block_size=self.block_size)


def _bits_to_bf16(t_np, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(t_np)).view(torch.bfloat16).to(device)


def upload(batch, device: str = "cuda") -> DeviceBatch:
    """Copy a seeded host batch (bf16 bit patterns, int32 tables) to the GPU."""
    import torch
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return DeviceBatch(q=_bits_to_bf16(batch.q, device), k_pool=_bits_to_bf16(batch.k_pool, device),
                       v_pool=_bits_to_bf16(batch.v_pool, device), page_table=i32(batch.page_table),
                       cu_seqlens=i32(batch.cu_seqlens), cu_qblocks=i32(batch.cu_qblocks),
                       total_qblocks=int(batch.cu_qblocks[-1]), seq_lens=tuple(batch.workload.seq_lens),
                       block_size=int(batch.block_size))


def upload_mask(order_mask: np.ndarray, mask_len: np.ndarray, device: str = "cuda"):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(order_mask, dtype=np.int32)).to(device),
            torch.from_numpy(np.ascontiguousarray(mask_len, dtype=np.int32)).to(device))


@dataclasses.dataclass
class PrefillOutputs:
    out: "torch.Tensor"
    lse: Optional["torch.Tensor"]
    decisions: Optional["torch.Tensor"]
    margins: Optional["torch.Tensor"]


def allocate_outputs(db: DeviceBatch, max_mask_len: int, log: bool) -> PrefillOutputs:
    import torch
    dev = db.q.device
    T, Hq = db.q.shape[0], db.q.shape[1]
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    dec = mar = None
    if log:
        dec = torch.empty((db.total_qblocks, Hq, max(max_mask_len, 1)), dtype=torch.uint8, device=dev)
        mar = torch.empty((db.total_qblocks, Hq, max(max_mask_len, 1)), dtype=torch.float32, device=dev)
    return PrefillOutputs(out, lse, dec, mar)


def workspace_for(db: DeviceBatch, max_mask_len: int):
    import torch
    n = binding.cosa_osk_workspace_bytes(db.dims(max_mask_len))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=db.q.device)


def abort_count(db: DeviceBatch, workspace, max_mask_len: int) -> int:
    """The workspace's health word after a completed call (0 when healthy)."""
    import torch
    n = binding.cosa_osk_workspace_bytes(db.dims(max_mask_len))
    return int(workspace[n - 256:n - 252].view(torch.int32).item())


def prefill(db: DeviceBatch, order_mask, mask_len, delta: float, log: bool = False,
            outputs: Optional[PrefillOutputs] = None, workspace=None, stream=None,
            sm_scale: float = 0.0, membership=None) -> PrefillOutputs:
    """One call of cosa_osk_prefill (cosa_osk_prefill_union with a membership mask) on
    device-resident inputs."""
    width = int(order_mask.shape[2])
    dims = db.dims(width, sm_scale)
    if outputs is None:
        outputs = allocate_outputs(db, width, log)
    if workspace is None:
        workspace = workspace_for(db, width)
    if membership is None:
        binding.cosa_osk_prefill(dims, db.q, db.k_pool, db.v_pool, db.page_table, db.cu_seqlens, db.cu_qblocks,
                                 order_mask, mask_len, delta, outputs.out, outputs.lse, outputs.decisions,
                                 outputs.margins, workspace=workspace, stream=stream)
    else:
        binding.cosa_osk_prefill_union(dims, db.q, db.k_pool, db.v_pool, db.page_table, db.cu_seqlens,
                                       db.cu_qblocks, order_mask, mask_len, membership, delta, outputs.out,
                                       outputs.lse, outputs.decisions, outputs.margins, workspace=workspace,
                                       stream=stream)
    return outputs


def build_mask(db: DeviceBatch, budget1: float, flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG,
               width: Optional[int] = None, scores: bool = False, workspace=None, stream=None):
    """cosa_build_order_mask on the device batch; returns (order_mask, mask_len[, scores])."""
    import torch
    max_pages = db.max_blocks
    if width is None:
        width = binding.cosa_order_mask_width(max_pages, budget1, flags)
    dims = db.dims(width)
    dev = db.q.device
    om = torch.empty((db.total_qblocks, db.num_kv_heads, width), dtype=torch.int32, device=dev)
    ml = torch.empty((db.total_qblocks, db.num_kv_heads), dtype=torch.int32, device=dev)
    sc = torch.empty((db.total_qblocks, db.num_kv_heads, max_pages), dtype=torch.float32, device=dev) if scores else None
    binding.cosa_build_order_mask(dims, db.q, db.k_pool, db.page_table, db.cu_seqlens, db.cu_qblocks, budget1,
                                  om, ml, flags=flags, proxy_scores=sc, workspace=workspace, stream=stream)
    return (om, ml, sc) if scores else (om, ml)


def build_kap_mask(db: DeviceBatch, stride: int, mode: int, budget: float, width: Optional[int] = None,
                   outputs: bool = False, workspace=None, stream=None, sm_scale: float = 0.0):
    """cosa_build_kap_mask on the device batch; returns (order_mask, mask_len[, scores, flags])."""
    import torch
    max_pages = db.max_blocks
    if width is None:
        width = binding.cosa_kap_mask_width(max_pages, mode, budget)
    dims = db.dims(width, sm_scale)
    dev = db.q.device
    om = torch.empty((db.total_qblocks, db.num_kv_heads, width), dtype=torch.int32, device=dev)
    ml = torch.empty((db.total_qblocks, db.num_kv_heads), dtype=torch.int32, device=dev)
    sc = torch.empty((db.total_qblocks, db.num_kv_heads, max_pages), dtype=torch.float32, device=dev) if outputs else None
    fl = torch.empty((db.total_qblocks, db.num_kv_heads, max_pages), dtype=torch.uint8, device=dev) if outputs else None
    binding.cosa_build_kap_mask(dims, db.q, db.k_pool, db.page_table, db.cu_seqlens, db.cu_qblocks, stride, mode,
                                budget, om, ml, kap_scores=sc, hrm_flags=fl, workspace=workspace, stream=stream)
    return (om, ml, sc, fl) if outputs else (om, ml)


def build_union_mask(db: DeviceBatch, budget1: float, flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG,
                     width: Optional[int] = None, workspace=None, stream=None):
    """cosa_build_union_mask; returns (order_mask, mask_len, membership, head_len)."""
    import torch
    G = db.num_q_heads // db.num_kv_heads
    if width is None:
        width = binding.cosa_union_mask_width(db.max_blocks, G, budget1, flags)
    dims = db.dims(width)
    dev = db.q.device
    om = torch.empty((db.total_qblocks, db.num_kv_heads, width), dtype=torch.int32, device=dev)
    ml = torch.empty((db.total_qblocks, db.num_kv_heads), dtype=torch.int32, device=dev)
    mem = torch.empty((db.total_qblocks, db.num_q_heads, width), dtype=torch.uint8, device=dev)
    hl = torch.empty((db.total_qblocks, db.num_q_heads), dtype=torch.int32, device=dev)
    binding.cosa_build_union_mask(dims, db.q, db.k_pool, db.page_table, db.cu_seqlens, db.cu_qblocks, budget1,
                                  om, ml, mem, hl, flags=flags, workspace=workspace, stream=stream)
    return om, ml, mem, hl


def validate_mask(db: DeviceBatch, order_mask, mask_len, stream=None) -> np.ndarray:
    """cosa_validate_order_mask; returns the 5 counters on the host."""
    import torch
    bad = torch.empty(5, dtype=torch.int32, device=db.q.device)
    binding.cosa_validate_order_mask(db.dims(int(order_mask.shape[2])), db.page_table, db.cu_seqlens,
                                     db.cu_qblocks, order_mask, mask_len, bad, stream=stream)
    return bad.cpu().numpy()


def dense_mask(db: DeviceBatch):
    """Every causal block 0..i in ascending order (the dense baseline's mask), built on the host."""
    rows = []
    for L in db.seq_lens:
        rows += list(range(-(-L // db.block_size)))
    width = max(rows) + 1
    om = np.full((db.total_qblocks, db.num_kv_heads, width), -1, dtype=np.int32)
    ml = np.zeros((db.total_qblocks, db.num_kv_heads), dtype=np.int32)
    for qb, i in enumerate(rows):
        om[qb, :, : i + 1] = np.arange(i + 1)
        ml[qb, :] = i + 1
    return upload_mask(om, ml, db.q.device)
