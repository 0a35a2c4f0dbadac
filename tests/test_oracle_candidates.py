"""Pins of the oracle's candidate-block scorer and top-k (the second level of a
two-level indexer: only the candidate blocks of each row are scored).

  - every block of a row as its candidates, in order, reproduces the dense logits on the
    valid cells and exactly the dense top-k (which its own pins tie to the definition);
  - on small rows, a brute-force enumeration written here (Python loops over the blocks
    and cells, sorted by value then token) gives the same top-k for random subsets;
  - padding block ids, ids past the page table, blocks past the valid length and rows
    with fewer valid cells than k behave as stated (no cells; -1 padding)."""
import numpy as np

import oracle
from sparse_attention_indexer_idx_amd import workloads as wl


def dense(W):
    pool = np.full(W.num_pages * W.page_stride_bytes + W.offset_bytes, 0xA5, np.uint8)
    oracle.k_store(pool, W.offset_bytes, W.page_stride_bytes, W.num_pages, W.page_size, oracle.FMT_MXFP4, W.k_rows,
                   W.gamma, W.eps, W.positions, W.cos_sin, W.slots)
    q, qs = oracle.q_quant_mxfp4(W.q_rows)
    return oracle.logits_paged(pool, W.offset_bytes, W.page_stride_bytes, W.num_pages, W.page_size,
                               oracle.FMT_MXFP4, q, qs, W.w, W.page_table, W.ctx, W.B, W.n_q, W.H, W.max_ctx)


def test_all_blocks_in_order_is_the_dense_path():
    W = wl.make_workload(0)
    d = dense(W)
    P, mp = W.page_size, W.page_table.shape[1]
    cand = np.tile(np.arange(mp, dtype=np.int32), (W.rows, 1))
    cl = oracle.logits_candidates(d, cand, P, mp, W.ctx, W.n_q)
    for r in range(W.rows):
        n = W.valid_len(r)
        assert np.array_equal(cl[r, :n], d[r, :n]) and np.all(np.isneginf(cl[r, n:]))
    for k in (1, 7, 64, 300):
        got = oracle.topk_candidates(cl, cand, P, mp, W.ctx, W.n_q, k)
        ref = oracle.topk(d, W.ctx, W.n_q, k)
        assert np.array_equal(got, ref)


def brute(d, cand, P, mp, W, k):
    out = np.full((W.rows, k), -1, np.int32)
    for r in range(W.rows):
        n = W.valid_len(r)
        items = []
        for cb in cand[r]:
            if cb < 0 or cb >= mp:
                continue
            for i in range(P):
                s = int(cb) * P + i
                if s < n:
                    items.append((-float(d[r, s]), s))
        items.sort()
        for t, (_, s) in enumerate(items[:k]):
            out[r, t] = s
    return out


def test_random_subsets_match_brute_force():
    W = wl.make_workload(0)
    d = dense(W)
    P, mp = W.page_size, W.page_table.shape[1]
    rng = np.random.default_rng(21)
    for trial in range(6):
        n_cand = int(rng.integers(1, mp + 1))
        cand = np.sort(np.stack([rng.choice(mp, n_cand, replace=False) for _ in range(W.rows)]), axis=1)
        cand = cand.astype(np.int32)
        if trial % 2:
            cand[:, -1] = -1           # a padding entry
        cl = oracle.logits_candidates(d, cand, P, mp, W.ctx, W.n_q)
        for k in (5, 64, 200):
            assert np.array_equal(oracle.topk_candidates(cl, cand, P, mp, W.ctx, W.n_q, k), brute(d, cand, P, mp, W, k))


def test_invalid_blocks_and_short_rows():
    W = wl.make_workload(0)              # ctx {200, 256}, page 64: row 0 has 4 blocks, the last partial
    d = dense(W)
    P, mp = W.page_size, W.page_table.shape[1]
    cand = np.array([[3, -1, mp, 7], [0, 1, -5, 2]], np.int32)
    cl = oracle.logits_candidates(d, cand, P, mp, W.ctx, W.n_q)
    n0 = W.valid_len(0)
    assert np.array_equal(cl[0, :n0 - 3 * P], d[0, 3 * P: n0])           # block 3 up to the valid length
    assert np.all(np.isneginf(cl[0, n0 - 3 * P:]))                      # the rest of row 0: no cells
    # row 1: blocks 0, 1, (padding), 2 -> cells [0, 2P) and [3P, 4P) hold tokens 0..2P-1, 2P..3P-1
    assert np.all(np.isfinite(cl[1, :2 * P])) and np.all(np.isneginf(cl[1, 2 * P: 3 * P]))
    assert np.array_equal(cl[1, 3 * P:], d[1, 2 * P: 3 * P])
    out = oracle.topk_candidates(cl, cand, P, mp, W.ctx, W.n_q, 100)
    assert np.all(out[0, :n0 - 3 * P] >= 3 * P) and np.all(out[0, n0 - 3 * P:] == -1)
    assert np.sum(out[1] >= 0) == 100 and set(out[1].tolist()) <= set(range(0, 3 * P))
