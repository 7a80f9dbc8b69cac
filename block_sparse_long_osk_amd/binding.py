"""ctypes binding of libcosa_osk.so: the C-ABI entry points under the same names.

Argument marshalling only -- every step of the computation runs in the HIP
library.  Tensors are torch tensors on the GPU (torch supplies device memory
and the stream).  A missing library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

# COSA_OSK_LIBRARY names another build of the same library (the host-sanitizer build
# that the host-only ABI tests run against); by default the in-tree build is used
LIB_PATH = os.environ.get("COSA_OSK_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libcosa_osk.so")

COSA_OK = 0
COSA_DECISION_COMPUTED, COSA_DECISION_SKIPPED, COSA_DECISION_NOT_VISITED = 0, 1, 2
COSA_FORCE_FIRST, COSA_FORCE_DIAG = 1, 2
COSA_KAP_FRACTION, COSA_KAP_TOP_P = 0, 1
PAGE_SIZE, HEAD_DIM = 64, 128


class CosaOskDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("total_q_tokens", ctypes.c_int32),
        ("total_qblocks", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32), ("max_mask_len", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("block_size", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("kv_stride_page", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64), ("kv_stride_tok", ctypes.c_int64),
    ]


class CosaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {cosa_status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_osk_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(CosaOskDims)
        L.cosa_abi_version.restype = ctypes.c_int
        L.cosa_abi_version.argtypes = []
        L.cosa_status_string.restype = ctypes.c_char_p
        L.cosa_status_string.argtypes = [ctypes.c_int]
        L.cosa_osk_workspace_bytes.restype = ctypes.c_size_t
        L.cosa_osk_workspace_bytes.argtypes = [D]
        L.cosa_osk_check_args.restype = ctypes.c_int
        L.cosa_osk_check_args.argtypes = [D, ctypes.c_size_t]
        L.cosa_osk_prefill.restype = ctypes.c_int
        L.cosa_osk_prefill.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, ctypes.c_size_t, P]
        L.cosa_osk_prefill_noalloc.restype = ctypes.c_int
        L.cosa_osk_prefill_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P]
        L.cosa_order_mask_width.restype = ctypes.c_int32
        L.cosa_order_mask_width.argtypes = [ctypes.c_int32, ctypes.c_float, ctypes.c_uint32]
        L.cosa_build_order_mask_workspace_bytes.restype = ctypes.c_size_t
        L.cosa_build_order_mask_workspace_bytes.argtypes = [D]
        L.cosa_build_order_mask.restype = ctypes.c_int
        L.cosa_build_order_mask.argtypes = [D, P, P, P, P, P, ctypes.c_float, ctypes.c_uint32, P, P, P, P,
                                            ctypes.c_size_t, P]
        L.cosa_kap_mask_width.restype = ctypes.c_int32
        L.cosa_kap_mask_width.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_float]
        L.cosa_build_kap_mask_workspace_bytes.restype = ctypes.c_size_t
        L.cosa_build_kap_mask_workspace_bytes.argtypes = [D]
        L.cosa_build_kap_mask.restype = ctypes.c_int
        L.cosa_build_kap_mask.argtypes = [D, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P, P, P,
                                          P, P, ctypes.c_size_t, P]
        L.cosa_validate_order_mask.restype = ctypes.c_int
        L.cosa_validate_order_mask.argtypes = [D, P, P, P, P, P, P, P]
        L.cosa_osk_prefill_union.restype = ctypes.c_int
        L.cosa_osk_prefill_union.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        L.cosa_union_mask_width.restype = ctypes.c_int32
        L.cosa_union_mask_width.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_uint32]
        L.cosa_build_union_mask_workspace_bytes.restype = ctypes.c_size_t
        L.cosa_build_union_mask_workspace_bytes.argtypes = [D]
        L.cosa_build_union_mask.restype = ctypes.c_int
        L.cosa_build_union_mask.argtypes = [D, P, P, P, P, P, ctypes.c_float, ctypes.c_uint32, P, P, P, P, P,
                                            ctypes.c_size_t, P]
        _lib = L
    return _lib


EXPORTED = ["cosa_abi_version", "cosa_status_string", "cosa_osk_workspace_bytes", "cosa_osk_check_args",
            "cosa_osk_prefill", "cosa_order_mask_width", "cosa_build_order_mask_workspace_bytes",
            "cosa_build_order_mask", "cosa_validate_order_mask", "cosa_kap_mask_width",
            "cosa_build_kap_mask_workspace_bytes", "cosa_build_kap_mask", "cosa_osk_prefill_union",
            "cosa_union_mask_width", "cosa_build_union_mask_workspace_bytes", "cosa_build_union_mask",
            "cosa_osk_prefill_noalloc"]
# bytes of the library-held scratch cosa_osk_prefill_noalloc uses (one copy per GPU)
COSA_OSK_NOALLOC_SCRATCH_BYTES = 66048


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != COSA_OK:
        raise CosaError(status, where)


# ----------------------------------------------------------------------------
# dims
# ----------------------------------------------------------------------------
def make_dims(q, k_pool, page_table, total_qblocks: int, max_mask_len: int, out=None,
              sm_scale: float = 0.0, block_size: int = 64) -> CosaOskDims:
    """Dims from tensor shapes/strides: q, out [T, Hq, 128]; pools [n_phys, Hkv, page_size, 128];
    page_table [S, max_pages]; logical blocks of block_size (64 or 128) tokens."""
    T, Hq, d = q.shape
    n_phys, Hkv, P, d2 = k_pool.shape
    out = q if out is None else out
    return CosaOskDims(
        num_seqs=page_table.shape[0], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=P,
        total_q_tokens=T, total_qblocks=int(total_qblocks), max_pages_per_seq=page_table.shape[1],
        num_phys_pages=n_phys, max_mask_len=int(max_mask_len), sm_scale=float(sm_scale), block_size=int(block_size),
        q_stride_tok=q.stride(0), q_stride_head=q.stride(1), o_stride_tok=out.stride(0),
        o_stride_head=out.stride(1), kv_stride_page=k_pool.stride(0), kv_stride_head=k_pool.stride(1),
        kv_stride_tok=k_pool.stride(2))


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------
def cosa_abi_version() -> int:
    return lib().cosa_abi_version()


def cosa_status_string(status: int) -> str:
    return lib().cosa_status_string(int(status)).decode()


def cosa_osk_workspace_bytes(dims: CosaOskDims) -> int:
    return lib().cosa_osk_workspace_bytes(ctypes.byref(dims))


def cosa_osk_check_args(dims: CosaOskDims, workspace_bytes: int) -> int:
    return lib().cosa_osk_check_args(ctypes.byref(dims), int(workspace_bytes))


def cosa_order_mask_width(max_pages_per_seq: int, budget1: float, flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG) -> int:
    return lib().cosa_order_mask_width(int(max_pages_per_seq), float(budget1), int(flags))


def cosa_build_order_mask_workspace_bytes(dims: CosaOskDims) -> int:
    return lib().cosa_build_order_mask_workspace_bytes(ctypes.byref(dims))


def cosa_osk_prefill(dims: CosaOskDims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask,
                     mask_len, budget2: float, out, lse=None, decisions=None, margins=None, workspace=None,
                     stream=None):
    """Launch the ordered-skipping prefill; workspace defaults to a fresh torch buffer."""
    if workspace is None:
        import torch
        workspace = torch.empty(max(cosa_osk_workspace_bytes(dims), 256), dtype=torch.uint8, device=q.device)
    st = lib().cosa_osk_prefill(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                _ptr(cu_seqlens), _ptr(cu_qblocks), _ptr(order_mask), _ptr(mask_len),
                                float(budget2), _ptr(out), _ptr(lse), _ptr(decisions), _ptr(margins),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "cosa_osk_prefill")


def cosa_osk_prefill_noalloc(dims: CosaOskDims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask,
                             mask_len, budget2: float, out, lse=None, decisions=None, margins=None, stream=None):
    """The prefill with the library-held scratch in place of a workspace (allocates nothing)."""
    st = lib().cosa_osk_prefill_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                        _ptr(cu_seqlens), _ptr(cu_qblocks), _ptr(order_mask), _ptr(mask_len),
                                        float(budget2), _ptr(out), _ptr(lse), _ptr(decisions), _ptr(margins),
                                        _stream(stream))
    _check(st, "cosa_osk_prefill_noalloc")


def cosa_build_order_mask(dims: CosaOskDims, q, k_pool, page_table, cu_seqlens, cu_qblocks, budget1: float,
                          order_mask, mask_len, flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG,
                          proxy_scores=None, workspace=None, stream=None):
    if workspace is None:
        import torch
        workspace = torch.empty(max(cosa_build_order_mask_workspace_bytes(dims), 256), dtype=torch.uint8,
                                device=q.device)
    st = lib().cosa_build_order_mask(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(page_table), _ptr(cu_seqlens),
                                     _ptr(cu_qblocks), float(budget1), int(flags), _ptr(order_mask), _ptr(mask_len),
                                     _ptr(proxy_scores), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "cosa_build_order_mask")


def cosa_kap_mask_width(max_pages_per_seq: int, mode: int, budget: float) -> int:
    return lib().cosa_kap_mask_width(int(max_pages_per_seq), int(mode), float(budget))


def cosa_build_kap_mask_workspace_bytes(dims: CosaOskDims) -> int:
    return lib().cosa_build_kap_mask_workspace_bytes(ctypes.byref(dims))


def cosa_build_kap_mask(dims: CosaOskDims, q, k_pool, page_table, cu_seqlens, cu_qblocks, stride: int, mode: int,
                        budget: float, order_mask, mask_len, kap_scores=None, hrm_flags=None, workspace=None,
                        stream=None):
    if workspace is None:
        import torch
        workspace = torch.empty(max(cosa_build_kap_mask_workspace_bytes(dims), 256), dtype=torch.uint8,
                                device=q.device)
    st = lib().cosa_build_kap_mask(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(page_table), _ptr(cu_seqlens),
                                   _ptr(cu_qblocks), int(stride), int(mode), float(budget), _ptr(order_mask),
                                   _ptr(mask_len), _ptr(kap_scores), _ptr(hrm_flags), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "cosa_build_kap_mask")


def cosa_validate_order_mask(dims: CosaOskDims, page_table, cu_seqlens, cu_qblocks, order_mask, mask_len,
                             bad_counts, stream=None):
    st = lib().cosa_validate_order_mask(ctypes.byref(dims), _ptr(page_table), _ptr(cu_seqlens), _ptr(cu_qblocks),
                                        _ptr(order_mask), _ptr(mask_len), _ptr(bad_counts), _stream(stream))
    _check(st, "cosa_validate_order_mask")


def cosa_osk_prefill_union(dims: CosaOskDims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask,
                           mask_len, membership, budget2: float, out, lse=None, decisions=None, margins=None,
                           workspace=None, stream=None):
    """The prefill with per-q-head membership of the union rows."""
    if workspace is None:
        import torch
        workspace = torch.empty(max(cosa_osk_workspace_bytes(dims), 256), dtype=torch.uint8, device=q.device)
    st = lib().cosa_osk_prefill_union(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                      _ptr(cu_seqlens), _ptr(cu_qblocks), _ptr(order_mask), _ptr(mask_len),
                                      _ptr(membership), float(budget2), _ptr(out), _ptr(lse), _ptr(decisions),
                                      _ptr(margins), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check(st, "cosa_osk_prefill_union")


def cosa_union_mask_width(max_blocks_per_seq: int, group: int, budget1: float,
                          flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG) -> int:
    return lib().cosa_union_mask_width(int(max_blocks_per_seq), int(group), float(budget1), int(flags))


def cosa_build_union_mask_workspace_bytes(dims: CosaOskDims) -> int:
    return lib().cosa_build_union_mask_workspace_bytes(ctypes.byref(dims))


def cosa_build_union_mask(dims: CosaOskDims, q, k_pool, page_table, cu_seqlens, cu_qblocks, budget1: float,
                          order_mask, mask_len, membership, head_len, flags: int = COSA_FORCE_FIRST | COSA_FORCE_DIAG,
                          workspace=None, stream=None):
    if workspace is None:
        import torch
        workspace = torch.empty(max(cosa_build_union_mask_workspace_bytes(dims), 256), dtype=torch.uint8,
                                device=q.device)
    st = lib().cosa_build_union_mask(ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(page_table), _ptr(cu_seqlens),
                                     _ptr(cu_qblocks), float(budget1), int(flags), _ptr(order_mask), _ptr(mask_len),
                                     _ptr(membership), _ptr(head_len), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "cosa_build_union_mask")
