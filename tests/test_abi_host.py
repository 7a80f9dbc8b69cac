"""The C-ABI library on the host: it loads, exports every declared symbol, and its
host-only argument checks return the documented status codes (no GPU calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_sparse_long_osk_amd import binding
from block_sparse_long_osk_amd.binding import CosaOskDims
from oracle.maskref import FORCE_DIAG, FORCE_FIRST, mask_width

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="library not built")


CALIB_LIB_PATH = os.path.join(os.path.dirname(binding.LIB_PATH), "libcosa_calib.so")


def declared_functions(headers):
    names = []
    for fn in headers:
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(cosa_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_every_header_is_checked():
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["cosa_calib.h", "cosa_osk.h"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    names = declared_functions(["cosa_osk.h"])
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(binding.EXPORTED) == names
    assert binding.cosa_abi_version() == 2
    assert binding.cosa_status_string(-3).startswith("workspace")


CHECKED_LIB_PATH = os.path.join(os.path.dirname(binding.LIB_PATH), "libcosa_osk_checked.so")


@pytest.mark.skipif(not os.path.exists(CHECKED_LIB_PATH), reason="bounds-checked library not built")
def test_checked_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(CHECKED_LIB_PATH)
    for n in declared_functions(["cosa_osk.h"]):
        assert hasattr(lib, n), n
    lib.cosa_abi_version.restype = ctypes.c_int
    assert lib.cosa_abi_version() == 2


@pytest.mark.skipif(not os.path.exists(CALIB_LIB_PATH), reason="calibration library not built")
def test_calibration_library_exports_and_host_checks():
    lib = ctypes.CDLL(CALIB_LIB_PATH)
    names = declared_functions(["cosa_calib.h"])
    assert names == ["cosa_calib_mfma_bf16", "cosa_calib_mfma_bf16_data", "cosa_calib_mfma_bf16_flop",
                     "cosa_calib_read"]
    for n in names:
        assert hasattr(lib, n), n
    lib.cosa_calib_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.cosa_calib_mfma_bf16_flop.restype = ctypes.c_double
    # 8 MFMAs of 32x32x16 multiply-adds per round, 4 waves per workgroup
    assert lib.cosa_calib_mfma_bf16_flop(3, 5) == 2 * 32 * 32 * 16 * 8 * 5 * 4 * 3
    # argument errors are caught on the host before any launch
    lib.cosa_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.cosa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_void_p]
    assert lib.cosa_calib_mfma_bf16(None, 1, 1, None) == -1
    assert lib.cosa_calib_mfma_bf16(ctypes.c_void_p(16), 0, 1, None) == -1
    lib.cosa_calib_mfma_bf16_data.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                              ctypes.c_void_p]
    assert lib.cosa_calib_mfma_bf16_data(None, 1, 2, 7, None) == -1
    assert lib.cosa_calib_mfma_bf16_data(ctypes.c_void_p(16), 0, 2, 7, None) == -1
    assert lib.cosa_calib_mfma_bf16_data(ctypes.c_void_p(16), 1, 3, 7, None) == -1  # odd round count
    assert lib.cosa_calib_read(None, 16, ctypes.c_void_p(16), 1, None) == -1
    assert lib.cosa_calib_read(ctypes.c_void_p(16), 17, ctypes.c_void_p(16), 1, None) == -1
    assert lib.cosa_calib_read(ctypes.c_void_p(24), 16, ctypes.c_void_p(16), 1, None) == -1


def good_dims(**kw):
    d = dict(num_seqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, total_q_tokens=4096,
             total_qblocks=64, max_pages_per_seq=64, num_phys_pages=64, max_mask_len=20, sm_scale=0.0,
             block_size=0, q_stride_tok=32 * 128, q_stride_head=128, o_stride_tok=32 * 128, o_stride_head=128,
             kv_stride_page=8 * 64 * 128, kv_stride_head=64 * 128, kv_stride_tok=128)
    d.update(kw)
    return CosaOskDims(**d)


def test_check_args_status_codes():
    d = good_dims()
    ws = binding.cosa_osk_workspace_bytes(d)
    assert ws >= 64 * 4
    assert binding.cosa_osk_check_args(d, ws) == OK
    assert binding.cosa_osk_check_args(d, ws - 256) == WORKSPACE
    assert binding.lib().cosa_osk_check_args(None, 1 << 20) == INVALID
    cases = [
        (dict(head_dim=64), UNSUPPORTED), (dict(page_size=128), UNSUPPORTED),
        (dict(num_q_heads=30), UNSUPPORTED), (dict(max_mask_len=-1), INVALID),
        (dict(max_mask_len=9000), UNSUPPORTED), (dict(total_qblocks=20000, total_q_tokens=20000 * 64), UNSUPPORTED),
        (dict(max_pages_per_seq=20000), UNSUPPORTED), (dict(num_kv_heads=0), INVALID),
        (dict(q_stride_head=100), INVALID), (dict(kv_stride_tok=0), INVALID),
        (dict(total_q_tokens=64 * 64 + 1), INVALID), (dict(total_qblocks=65, total_q_tokens=64), INVALID),
        (dict(block_size=1), UNSUPPORTED), (dict(block_size=256), UNSUPPORTED), (dict(block_size=64), OK),
        # 128-token blocks: pages of 16 .. 128 tokens; blocks of up to 128 query tokens
        (dict(block_size=128, total_qblocks=32), OK), (dict(block_size=128, page_size=128, total_qblocks=32), OK),
        (dict(block_size=128, page_size=16, total_qblocks=32), OK),
        (dict(block_size=128, total_qblocks=31), INVALID),
        (dict(block_size=128, page_size=256, total_qblocks=32), UNSUPPORTED),
        (dict(sm_scale=float("nan")), INVALID),
        (dict(kv_stride_tok=(1 << 24) + 8), UNSUPPORTED), (dict(kv_stride_tok=1 << 24), OK),
    ]
    for kw, want in cases:
        dd = good_dims(**kw)
        assert binding.cosa_osk_check_args(dd, 1 << 30) == want, kw


def test_prefill_rejects_bad_arguments_before_launch():
    """Null / misaligned pointers, missing workspace, margins without decisions and
    a NaN skip scale are refused on the host (nothing is launched)."""
    L = binding.lib()
    d = good_dims()
    ws = binding.cosa_osk_workspace_bytes(d)
    fake = 0x10000  # never dereferenced: checks fail first
    args = [fake] * 8
    def call(q=fake, out=fake, dec=None, mar=None, work=fake, wsb=ws, budget=1.0, mask=fake):
        return L.cosa_osk_prefill(ctypes.byref(d), q, fake, fake, fake, fake, fake, mask, fake, budget, out,
                                  None, dec, mar, work, wsb, None)
    assert call(q=None) == INVALID
    assert call(out=fake + 2) == INVALID
    assert call(mask=None) == INVALID
    assert call(mar=fake) == INVALID
    assert call(budget=float("nan")) == INVALID
    assert call(work=None) == WORKSPACE
    assert call(wsb=0) == WORKSPACE
    assert L.cosa_osk_prefill(None, *([None] * 8), 1.0, None, None, None, None, None, 0, None) == INVALID


@pytest.mark.parametrize("max_pages,b1,flags", [(32, 0.5, 3), (256, 0.25, 3), (512, 0.2, 3), (2048, 0.1, 3),
                                                (100, 0.3, FORCE_FIRST), (77, 0.15, FORCE_DIAG), (5, 1.0, 0),
                                                (1, 0.5, 3), (2, 0.0, 3)])
def test_mask_width_matches_oracle(max_pages, b1, flags):
    assert binding.cosa_order_mask_width(max_pages, b1, flags) == mask_width(max_pages, float(np.float32(b1)), flags)


def test_builder_rejects_bad_arguments():
    L = binding.lib()
    d = good_dims(max_mask_len=5)
    fake = 0x10000
    need = binding.cosa_build_order_mask_workspace_bytes(d)
    assert need >= 2 * 64 * 8 * 128 * 4
    def call(dd=d, b1=0.1, flags=3, wsb=need, work=fake):
        return L.cosa_build_order_mask(ctypes.byref(dd), fake, fake, fake, fake, fake, b1, flags, fake, fake,
                                       None, work, wsb, None)
    assert call(b1=1.5) == INVALID
    assert call(flags=4) == INVALID
    assert call(dd=good_dims(max_mask_len=3)) == INVALID          # narrower than the mask needs
    assert call(dd=good_dims(max_mask_len=20), wsb=16) == WORKSPACE
    assert call(dd=good_dims(max_mask_len=20, max_pages_per_seq=9000, total_qblocks=64)) == UNSUPPORTED


def test_kap_mask_width_matches_oracle():
    from oracle import kap
    for mode, b in [(0, 0.1), (0, 0.3), (0, 1.0), (1, 0.95), (1, 0.0)]:
        for mp in (1, 3, 64, 2048, 8192):
            assert binding.cosa_kap_mask_width(mp, mode, b) == kap.mask_width(mp, mode, b), (mode, b, mp)
    assert binding.cosa_kap_mask_width(0, 0, 0.5) == -1
    assert binding.cosa_kap_mask_width(64, 2, 0.5) == -1


def test_kap_builder_rejects_bad_arguments():
    L = binding.lib()
    d = good_dims(max_mask_len=64)
    fake = 0x10000
    need = binding.cosa_build_kap_mask_workspace_bytes(d)
    # scores and flags [64 query blocks, 8 KV heads, 64 blocks], uint32 row maxima of 32 q
    # heads x up to 8 sampled rows per query block, 8 KV heads x (64 / 4 + 1) key tiles
    assert need >= 64 * 8 * 64 * 5 + 64 * 32 * 8 * 4 + 8 * (64 // 4 + 1) * 8192
    def call(dd=d, stride=16, mode=0, b=0.3, wsb=need, work=fake):
        return L.cosa_build_kap_mask(ctypes.byref(dd), fake, fake, fake, fake, fake, stride, mode, b, fake, fake,
                                     None, None, work, wsb, None)
    assert call(mode=2) == INVALID
    assert call(b=0.0) == INVALID                                   # a fixed fraction of zero keeps nothing
    assert call(mode=1, b=1.5) == INVALID
    assert call(stride=32) == UNSUPPORTED
    assert call(stride=4) == UNSUPPORTED
    assert call(dd=good_dims(num_q_heads=24, max_mask_len=64)) == UNSUPPORTED      # G = 3: 12 rows per block
    assert call(dd=good_dims(num_q_heads=64, max_mask_len=64), stride=8) == UNSUPPORTED  # G = 8 at stride 8: 64 rows
    assert call(dd=good_dims(max_mask_len=10)) == INVALID          # narrower than the mask needs
    assert call(mode=1, dd=good_dims(max_mask_len=63)) == INVALID  # Top-p rows can hold every candidate
    assert call(wsb=16) == WORKSPACE
    assert call(dd=good_dims(max_mask_len=64, max_pages_per_seq=9000)) == UNSUPPORTED
    # 128-token blocks: strides 32 and 16 give 4 and 8 samples per block, 8 gives 16.  An
    # accepted stride reaches the workspace check (too small here: nothing is launched)
    d128 = good_dims(max_mask_len=64, block_size=128, total_qblocks=32)
    assert call(dd=d128, stride=32, wsb=16) == WORKSPACE
    assert call(dd=d128, stride=16, wsb=16) == WORKSPACE
    assert call(dd=d128, stride=8, wsb=16) == UNSUPPORTED
    assert call(dd=d128, stride=48, wsb=16) == UNSUPPORTED
    assert call(stride=16, wsb=16) == WORKSPACE and call(stride=8, wsb=16) == WORKSPACE


def test_union_mask_width_matches_oracle():
    from oracle.maskref import union_mask_width
    for mp, G, b1, flags in [(32, 4, 0.5, 3), (2048, 4, 0.1, 3), (100, 2, 0.3, FORCE_FIRST), (7, 8, 1.0, 0),
                             (1, 4, 0.5, 3), (300, 1, 0.2, 3)]:
        want = union_mask_width(mp, G, float(np.float32(b1)), flags)
        assert binding.cosa_union_mask_width(mp, G, b1, flags) == want, (mp, G, b1, flags)
    assert binding.cosa_union_mask_width(0, 4, 0.5, 3) == -1
    assert binding.cosa_union_mask_width(8, 0, 0.5, 3) == -1


def test_union_entry_points_reject_bad_arguments_before_launch():
    L = binding.lib()
    fake = 0x10000
    d = good_dims()
    ws = binding.cosa_osk_workspace_bytes(d)
    # the union prefill needs a membership mask whenever rows have entries
    assert L.cosa_osk_prefill_union(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, None, 1.0,
                                    fake, None, None, None, fake, ws, None) == INVALID
    # and otherwise checks as the prefill does (here: a workspace that is too small)
    assert L.cosa_osk_prefill_union(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, fake, 1.0,
                                    fake, None, None, None, fake, 0, None) == WORKSPACE
    G = 4
    width = binding.cosa_union_mask_width(64, G, 0.2, 3)
    du = good_dims(max_mask_len=width)
    need = binding.cosa_build_union_mask_workspace_bytes(du)
    assert need > binding.cosa_build_order_mask_workspace_bytes(du)
    def call(dd=du, b1=0.2, flags=3, mem=fake, hl=fake, wsb=need, work=fake):
        return L.cosa_build_union_mask(ctypes.byref(dd), fake, fake, fake, fake, fake, b1, flags, fake, fake, mem, hl,
                                       work, wsb, None)
    assert call(mem=None) == INVALID
    assert call(hl=None) == INVALID
    assert call(b1=-0.5) == INVALID
    assert call(flags=8) == INVALID
    assert call(dd=good_dims(max_mask_len=width - 1)) == INVALID          # narrower than the union can be
    assert call(wsb=need - 1) == WORKSPACE
    assert call(dd=good_dims(num_q_heads=40 * 8, max_mask_len=64 * 40)) == UNSUPPORTED   # 40 heads per group


def test_empty_batch_needs_no_pointers_or_workspace():
    """total_qblocks = 0 (every sequence empty): the prefill and builder entry points check
    dims and their scalar arguments, launch nothing and return OK with NULL pointers and
    no workspace (nothing is read or written); scalar errors are still reported."""
    L = binding.lib()
    d = good_dims(num_seqs=2, total_q_tokens=0, total_qblocks=0, max_mask_len=64)
    nul = [None] * 8
    assert L.cosa_osk_prefill(ctypes.byref(d), *nul, 1.0, None, None, None, None, None, 0, None) == OK
    assert L.cosa_osk_prefill_noalloc(ctypes.byref(d), *nul, 1.0, None, None, None, None, None) == OK
    assert L.cosa_osk_prefill_union(ctypes.byref(d), *nul, None, 1.0, None, None, None, None, None, 0,
                                    None) == OK
    assert L.cosa_osk_prefill(ctypes.byref(d), *nul, float("nan"), None, None, None, None, None, 0,
                              None) == INVALID
    assert L.cosa_osk_prefill(ctypes.byref(d), *nul, 1.0, None, None, None, 0x10000, None, 0, None) == INVALID
    def build(b1=0.1):
        return L.cosa_build_order_mask(ctypes.byref(d), None, None, None, None, None, b1, 3, None, None, None,
                                       None, 0, None)
    assert build() == OK
    assert build(b1=1.5) == INVALID
    assert L.cosa_build_union_mask(ctypes.byref(d), None, None, None, None, None, 0.1, 3, None, None, None, None,
                                   None, 0, None) == OK
    def kap(stride=16):
        return L.cosa_build_kap_mask(ctypes.byref(d), None, None, None, None, None, stride, 0, 0.1, None, None,
                                     None, None, None, 0, None)
    assert kap() == OK
    assert kap(stride=12) == UNSUPPORTED
    # the strides of an empty Q / output and of an empty pool are not checked (zero-element
    # arrays often carry zero strides); a non-empty one still needs valid strides
    dz = good_dims(num_seqs=2, total_q_tokens=0, total_qblocks=0, q_stride_tok=0, q_stride_head=0,
                   o_stride_tok=0, o_stride_head=0, max_mask_len=64)
    assert L.cosa_osk_prefill(ctypes.byref(dz), *nul, 1.0, None, None, None, None, None, 0, None) == OK
    assert binding.cosa_osk_check_args(good_dims(q_stride_tok=0), 1 << 20) == INVALID
    assert binding.cosa_osk_check_args(good_dims(num_phys_pages=0, kv_stride_page=0, kv_stride_head=0,
                                                 kv_stride_tok=0), 1 << 20) == OK
    assert binding.cosa_osk_check_args(good_dims(kv_stride_tok=0), 1 << 20) == INVALID
    # a page table of no columns is accepted for an empty batch only
    d0 = good_dims(num_seqs=2, total_q_tokens=0, total_qblocks=0, max_pages_per_seq=0, max_mask_len=0)
    assert L.cosa_osk_prefill(ctypes.byref(d0), *nul, 1.0, None, None, None, None, None, 0, None) == OK
    assert binding.cosa_osk_check_args(good_dims(max_pages_per_seq=0), 1 << 20) == INVALID
    bad = good_dims(num_seqs=2, total_q_tokens=0, total_qblocks=0, head_dim=64)
    assert L.cosa_osk_prefill(ctypes.byref(bad), *nul, 1.0, None, None, None, None, None, 0, None) == UNSUPPORTED
