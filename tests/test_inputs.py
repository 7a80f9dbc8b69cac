"""The seeded input generator: bfloat16 rounding, determinism and layouts (no GPU)."""
import numpy as np
import pytest

from block_sparse_long_osk_amd import inputs
from block_sparse_long_osk_amd.inputs import PAGE, bf16_bits_to_f32, f32_to_bf16_bits


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)           # bf16 spacing just above 1
    xs = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0, 3.0e-39],
                  dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(xs))
    want = np.array([1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0 + ulp, -2.5, 0.0, np.nan], dtype=np.float32)
    np.testing.assert_array_equal(got[:6], want[:6])
    assert abs(got[6] - 3.0e-39) < 2.0 ** -133 * 2 ** 7      # subnormals round too
    assert one == 1.0


def test_generator_is_deterministic_and_shaped():
    wl = inputs.small_workload("t", [130, 64], 8, 2, generator="structured", pool="shuffled", budget1=0.3)
    a = inputs.generate(wl)
    b = inputs.generate(wl)
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.page_table, b.page_table)]:
        assert np.array_equal(x, y)
    assert a.q.shape == (194, 8, 128) and a.q.dtype == np.uint16
    assert a.k_pool.shape[1:] == (2, PAGE, 128)
    assert list(a.cu_seqlens) == [0, 130, 194] and list(a.cu_qblocks) == [0, 3, 4]
    used = a.page_table[a.page_table >= 0]
    assert len(set(used.tolist())) == used.size                     # pages are distinct
    # tail slots of the last page of sequence 0 (130 = 2*64 + 2) stay zero
    tail = a.k_pool[a.page_table[0, 2], :, 2:, :]
    assert (tail == 0).all()


def test_structured_planting_is_visible_in_logits():
    """Salient and sink pages carry +3 u_g along the group's query direction."""
    wl = inputs.small_workload("t", [64 * 40], 4, 1, generator="structured", seed=3)
    bt = inputs.generate(wl)
    q = bf16_bits_to_f32(bt.q).astype(np.float64)
    k = bf16_bits_to_f32(bt.k_pool).astype(np.float64)
    qbar = q[-64:, :, :].mean(axis=(0, 1))
    page_mean = k[:, 0].mean(axis=1) @ qbar                         # [n_pages]
    sal = set(bt.salient_pages[0][0].tolist()) | {0}
    others = [j for j in range(36) if j not in sal]                 # exclude the local window 36..39
    assert min(page_mean[j] for j in sal) > max(page_mean[j] for j in others)


@pytest.mark.parametrize("bp", [16, 32, 128])
def test_repage_is_a_storage_change_only(bp):
    from oracle import paging
    wl = inputs.small_workload("rp", [64 * 6 + 17, 64 * 2, 5], 4, 2, generator="structured", seed=3, pool="shuffled")
    bt = inputs.generate(wl)
    rp = inputs.repage(bt, bp, 11)
    assert rp.k_pool.shape[2] == bp
    B = max(64, bp)   # the logical view at a block size both layouts divide
    kl, vl, ptl = paging.logical_view(rp.k_pool, rp.v_pool, rp.page_table, rp.cu_seqlens, bp, block=B)
    k0, v0, pt0 = paging.logical_view(bt.k_pool, bt.v_pool, bt.page_table, bt.cu_seqlens, 64, block=B)
    np.testing.assert_array_equal(ptl, pt0)
    np.testing.assert_array_equal(kl, k0)
    np.testing.assert_array_equal(vl, v0)
    # every physical page is used at most once
    used = rp.page_table[rp.page_table >= 0]
    assert used.size == np.unique(used).size


def test_block128_workload_counts_128_token_blocks():
    import dataclasses
    wl = inputs.small_workload("b", [128 * 5 + 3, 64, 129], 4, 2, generator="iid", seed=2, pool="shuffled")
    bt64 = inputs.generate(wl)
    bt = inputs.generate(dataclasses.replace(wl, block_size=128))
    assert list(bt.cu_qblocks) == [0, 6, 7, 9] and bt.block_size == 128
    assert bt.max_blocks == -(-bt.max_pages * 64 // 128)
    # the same tokens and pages as the 64-token workload
    np.testing.assert_array_equal(bt.k_pool, bt64.k_pool)
    np.testing.assert_array_equal(bt.page_table, bt64.page_table)
    wl128 = inputs.WORKLOADS["cfg4_128k_structured_b128"]
    assert wl128.block_size == 128 and wl128.page_size == 64 and wl128.seq_lens == (131072,)
