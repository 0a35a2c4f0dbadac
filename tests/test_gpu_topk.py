"""GPU parity: per-row top-k.

Isolated: on the same fp32 logits (seeded draws, with and without heavy ties) the
HIP top-k and the oracle select exactly the same index sets — the decision is taken in
fp32 on both sides.  End to end: GPU scorer + GPU top-k against oracle logits (fp64) +
the tolerance rule (clear winners in, clear losers out, exact sizes and padding)."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G
from tests.test_gpu_logits import run_scorer, setup_scorer

pytestmark = pytest.mark.gpu


def gpu_topk(logits_d, ctx, B, n_q, max_ctx, k):
    torch = G.torch_cuda()
    out = torch.full((B * n_q, k), -5, dtype=torch.int32, device="cuda")
    bd.idx_topk(logits_d, G.dev(np.asarray(ctx, np.int32)), B, n_q, max_ctx, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows,n_q,lens,k,ties", [
    (64, 1, (8192, 8192), 1024, False),      # decode shape
    (64, 1, (8192, 8192), 1024, True),
    (8, 1, (1000, 3000), 1024, False),       # around k
    (6, 3, (1020, 1030), 1024, True),        # n_q > 1, rows either side of k
    (3000, 1, (1, 8192), 1024, False),       # many rows: the 256-thread variant
    (3000, 1, (1025, 4000), 1024, True),
    (4, 1, (65536, 65536), 1024, False),     # the longest supported row
    (5, 1, (300, 301), 7, True),             # small k
    (4, 2, (0, 3), 4, False),                # empty and tiny rows
])
def test_topk_isolated_exact(rows, n_q, lens, k, ties):
    rng = np.random.default_rng(rows * 7 + k + int(ties))
    B = rows // n_q
    ctx = rng.integers(lens[0], lens[1] + 1, B).astype(np.int32)
    stride = int(ctx.max()) + 5
    lg = wl.random_logits(rng, B * n_q, stride, ties=ties)
    G.say(f"topk isolated rows={B * n_q} n_q={n_q} ctx={lens} k={k} ties={ties}")
    got = gpu_topk(G.dev(lg), ctx, B, n_q, int(ctx.max()), k)
    ref = oracle.topk(lg, ctx, n_q, k)
    for r in range(B * n_q):
        g, o = got[r], ref[r]
        assert np.array_equal(np.sort(g[g >= 0]), np.sort(o[o >= 0])), f"row {r}"
        m = int((o >= 0).sum())
        assert np.all(g[m:] == -1) and np.all(g[:m] >= 0)
        assert np.all(np.diff(g[:m]) > 0)  # ascending index order


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_score_plus_topk_end_to_end(cfg):
    torch = G.torch_cuda()
    W = wl.make_workload(cfg)
    G.say(f"score+topk cfg={cfg}")
    d = setup_scorer(W, wl.MXFP4)
    logits = run_scorer(W, d)
    got = gpu_topk(logits, W.ctx, W.B, W.n_q, W.max_ctx, W.topk)
    rows = np.arange(W.rows)
    ref = G.oracle_logits(d["hp"], d["q"], d["qs"], d["w"], rows, W.max_ctx)
    mask = G.valid_mask(W, rows, W.max_ctx)
    tau = 1e-4 * np.abs(ref[mask]).max()
    G.assert_topk_valid(got, ref, W, rows, W.topk, tau, f"cfg{cfg}")
    del torch


def test_score_plus_topk_prefill_sampled():
    W = wl.make_workload(2)
    G.say("score+topk cfg=2 sampled")
    d = setup_scorer(W, wl.MXFP4)
    logits = run_scorer(W, d)
    got_all = gpu_topk(logits, W.ctx, W.B, W.n_q, W.max_ctx, W.topk)
    rows = np.array([0, 5, 1022, 1023, 1024, 1025, 2047, 5000, 8191])
    ref = G.oracle_logits(d["hp"], d["q"], d["qs"], d["w"], rows, W.max_ctx)
    tau = 1e-4 * np.nanmax(np.abs(ref))
    G.assert_topk_valid(got_all[rows], ref, W, rows, W.topk, tau, "cfg2")


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_score_plus_topk_large_pool_sampled(fmt):
    W = wl.make_workload(4, kv_format=fmt)
    G.say(f"score+topk cfg=4 fmt={fmt} sampled")
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d)
    got_all = gpu_topk(logits, W.ctx, W.B, W.n_q, W.max_ctx, W.topk)
    rows = np.array([0, 17, 100, 255])
    ref = G.oracle_logits(d["hp"], d["q"], d["qs"], d["w"], rows, W.max_ctx)
    tau = 1e-4 * np.nanmax(np.abs(ref))
    G.assert_topk_valid(got_all[rows], ref, W, rows, W.topk, tau, f"cfg4/fmt{fmt}")
