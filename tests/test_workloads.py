"""The seeded input generators: shapes, page maps and address-boundary coverage."""
import numpy as np
import pytest

from sparse_attention_indexer_idx_amd import workloads as wl


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_page_tables_are_distinct_and_in_pool(cfg):
    W = wl.make_workload(cfg)
    used = W.page_table[W.page_table >= 0]
    assert used.size == len(set(used.tolist())) and used.max() < W.num_pages
    for b in range(W.B):
        need = (int(W.ctx[b]) + W.page_size - 1) // W.page_size
        assert np.all(W.page_table[b, :need] >= 0) and np.all(W.page_table[b, need:] == -1)
    assert W.page_stride_bytes >= W.page_bytes and W.page_stride_bytes % 256 == 0 and W.offset_bytes % 256 == 0
    assert W.k_rows.shape == (int(W.ctx.sum()), 128) and W.q_rows.shape == (W.B, W.n_q, W.H, 128)
    assert np.all(W.slots // W.page_size == W.page_table[W.k_seq, W.positions // W.page_size])


def test_shapes_of_the_five_workloads():
    W0 = wl.make_workload(0)
    assert (W0.B, W0.n_q, W0.H, W0.page_size, W0.topk, W0.num_pages) == (2, 1, 4, 64, 64, 16)
    assert list(W0.ctx) == [200, 256]
    W3 = wl.make_workload(3)
    assert (W3.B, W3.n_q, W3.H, W3.page_size) == (128, 3, 64, 64)
    assert W3.ctx.min() >= 256 and W3.ctx.max() <= 2368 and W3.offset_bytes > 0
    assert W3.page_stride_bytes > W3.page_bytes


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    got = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x))
    assert list(got[:4]) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5]


def test_large_pool_straddles_address_boundaries():
    for fmt, stride, want in ((wl.MXFP4, 68 * 128, [246723, 493447, 555128, 529411]),
                              (wl.FP8, 132 * 128, [127100, 254200, 285975, 272727])):
        pids = wl.straddling_pages(stride)
        assert pids == want
        for pid, boundary in zip(pids, (1 << 31, 1 << 32, 4608 << 20, 4_608_000_000)):
            assert pid * stride < boundary < (pid + 1) * stride


@pytest.mark.slow
def test_large_pool_workload_includes_straddling_pages():
    W = wl.make_workload(4, scale={"B": 8})
    used = set(W.page_table[W.page_table >= 0].tolist())
    assert set(wl.straddling_pages(W.page_stride_bytes)) <= used
    assert W.pool_bytes <= 6 * wl.GIB and W.num_pages == (6 * wl.GIB) // (68 * 128)
