"""GPU parity: the candidate-block scorer and its top-k against the oracle.

A row scores only its candidate blocks (page-table indices of its sequence); every cell
of the candidate layout is written, -inf where the cell is not a valid candidate.  K bytes
and packed Q come from the oracle.  Logits: valid cells within max|d| <= 1e-4 * max|ref|
and cosine >= 0.999999 of the oracle, every other cell exactly -inf.  Top-k: on the same
fp32 input (seeded draws) the HIP and oracle selections are equal sets; end to end, the
tolerance rule against fp64 logits."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G
from tests.test_gpu_logits import setup_scorer

pytestmark = pytest.mark.gpu


def run_cand(W, d, cand, stride=None):
    torch = G.torch_cuda()
    stride = stride or cand.shape[1] * W.page_size
    logits = torch.empty((W.rows, stride), dtype=torch.float32, device="cuda")
    logits.view(torch.int32).fill_(np.int32(np.uint32(G.SENTINEL_BITS).view(np.int32)))
    bd.idx_logits_candidates(d["pool"].view, d["q_d"], d["qs_d"], d["w_d"], d["pt_d"], d["ctx_d"], W.B, W.n_q, W.H,
                             G.dev(cand), logits)
    torch.cuda.synchronize()
    return logits


def gpu_topk_cand(logits_d, cand, P, B, n_q, k):
    torch = G.torch_cuda()
    out = torch.full((B * n_q, k), -5, dtype=torch.int32, device="cuda")
    bd.idx_topk_candidates(logits_d, G.dev(cand), P, B, n_q, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_cand(W, d, cand, rows):
    """Oracle candidate logits of `rows` (dense oracle logits of those rows' sequences)."""
    dense = np.full((W.rows, W.max_ctx), np.nan)
    dense[rows] = G.oracle_logits(d["hp"], d["q"], d["qs"], d["w"], rows, W.max_ctx)
    return oracle.logits_candidates(dense, cand, W.page_size, W.page_table.shape[1], W.ctx, W.n_q)[rows]


def check_cand(W, d, cand, logits, rows, label):
    n_cells = cand.shape[1] * W.page_size
    got = logits.cpu().numpy()[rows]
    ref = oracle_cand(W, d, cand, rows)
    valid = np.isfinite(ref)
    stats = G.assert_logits_close(got[:, :n_cells], ref, valid, label)
    assert np.all(np.isneginf(got[:, :n_cells][~valid])), f"{label}: a non-candidate cell is not -inf"
    assert np.all(got[:, n_cells:].view(np.uint32) == G.SENTINEL_BITS), f"{label}: a cell past the candidates written"
    G.say(f"{label}: {stats}, valid cells {int(valid.sum())}")
    return ref


def check_topk_cand(W, cand, got, ref, rows, k, label):
    """Tolerance rule over candidate cells (ref: oracle fp64 candidate logits of `rows`)."""
    tau = 1e-4 * np.abs(ref[np.isfinite(ref)]).max()
    tok, ok = oracle.candidate_cells(cand, W.page_size, W.page_table.shape[1], W.ctx, W.n_q)
    for i, r in enumerate(rows):
        vt, vv = tok[r][ok[r]], ref[i][ok[r]]
        m = min(k, vt.size)
        sel = got[i]
        assert np.all(sel[:m] >= 0) and np.all(sel[m:] == -1), f"{label} row {r}: padding"
        s = set(sel[:m].tolist())
        assert len(s) == m and s <= set(vt.tolist()), f"{label} row {r}: duplicates or non-candidates"
        if vt.size <= k:
            continue
        vk = np.sort(vv)[::-1][k - 1]
        assert set(vt[vv > vk + tau].tolist()) <= s, f"{label} row {r}: missing a clear winner"
        assert not (set(vt[vv < vk - tau].tolist()) & s), f"{label} row {r}: selected a clear loser"


@pytest.mark.parametrize("cfg,fmt,n_cand,pad,past,shuffled", [
    (0, wl.MXFP4, 3, 0, 0, False),
    (0, wl.MXFP4, 4, 1, 1, True),     # padding, ids past the table, unsorted ids
    (0, wl.FP8, 4, 1, 0, False),
    (3, wl.MXFP4, 20, 2, 1, False),    # n_q 3, 64 heads, page 64: blocks past the valid length
    (3, wl.FP8, 8, 0, 0, True),
])
def test_candidates_all_rows(cfg, fmt, n_cand, pad, past, shuffled):
    W = wl.make_workload(cfg, kv_format=fmt)
    rng = np.random.default_rng(300 + 10 * cfg + n_cand)
    cand = wl.candidate_blocks(rng, W, n_cand, pad=pad, past_table=past, shuffled=shuffled)
    G.say(f"candidates cfg={cfg} fmt={fmt} n_cand={n_cand} pad={pad} past={past} shuffled={shuffled}")
    d = setup_scorer(W, fmt)
    logits = run_cand(W, d, cand, stride=cand.shape[1] * W.page_size + 7)
    rows = np.arange(W.rows)
    ref = check_cand(W, d, cand, logits, rows, f"cand cfg{cfg}/fmt{fmt}")
    for k in (1, 64, W.topk):
        got = gpu_topk_cand(logits, cand, W.page_size, W.B, W.n_q, k)
        check_topk_cand(W, cand, got, ref, rows, k, f"cand topk cfg{cfg} k={k}")


def test_candidates_decode_sampled_rows():
    W = wl.make_workload(1)
    rng = np.random.default_rng(311)
    cand = wl.candidate_blocks(rng, W, 16)   # 16 of 64 blocks: 2048 cells per row
    G.say("candidates cfg=1 (B64/H32/8K, 16 blocks of 128), sampled rows")
    d = setup_scorer(W, wl.MXFP4)
    logits = run_cand(W, d, cand)
    rows = np.array([0, 1, 17, 40, 63])
    ref = check_cand(W, d, cand, logits, rows, "cand cfg1")
    got = gpu_topk_cand(logits, cand, W.page_size, W.B, W.n_q, W.topk)[rows]
    check_topk_cand(W, cand, got, ref, rows, W.topk, "cand topk cfg1")


def test_candidates_no_candidates_and_all_padding():
    W = wl.make_workload(0)
    d = setup_scorer(W, wl.MXFP4)
    G.say("candidates: n_cand 0 and all padding")
    cand = np.full((W.rows, 2), -1, np.int32)
    logits = run_cand(W, d, cand)
    assert np.all(np.isneginf(logits.cpu().numpy()))
    assert np.all(gpu_topk_cand(logits, cand, W.page_size, W.B, W.n_q, 5) == -1)
    torch = G.torch_cuda()
    empty = np.zeros((W.rows, 0), np.int32)
    lg = torch.zeros((W.rows, 8), dtype=torch.float32, device="cuda")
    bd.idx_logits_candidates(d["pool"].view, d["q_d"], d["qs_d"], d["w_d"], d["pt_d"], d["ctx_d"], W.B, W.n_q, W.H,
                             G.dev(np.zeros((W.rows, 1), np.int32))[:, :0], lg)
    assert np.all(gpu_topk_cand(lg, empty, W.page_size, W.B, W.n_q, 3) == -1)
    torch.cuda.synchronize()
    assert np.all(lg.cpu().numpy() == 0.0)


@pytest.mark.parametrize("rows,n_cand,P,k,ties", [
    (64, 16, 128, 1024, False),
    (64, 16, 128, 1024, True),
    (700, 8, 64, 300, False),      # many rows: a smaller block size
    (5, 3, 16, 7, True),
    (3, 512, 128, 1024, False),    # the longest supported row (65536 cells)
])
def test_topk_candidates_isolated_exact(rows, n_cand, P, k, ties):
    """Same fp32 input on both sides: ascending distinct ids, a few padding entries, and
    -inf in the cells a candidate scorer would mark invalid."""
    rng = np.random.default_rng(rows + n_cand + k + int(ties))
    mp = 2 * n_cand + 3
    cand = np.stack([np.sort(rng.choice(mp, n_cand, replace=False)) for _ in range(rows)]).astype(np.int32)
    cand[rng.random(cand.shape) < 0.1] = -1
    lg = wl.random_logits(rng, rows, n_cand * P, ties=ties)
    ctx = np.full(rows, mp * P, np.int32)
    tok, ok = oracle.candidate_cells(cand, P, mp, ctx, 1)
    lg[~ok] = -np.inf
    G.say(f"topk candidates isolated rows={rows} n_cand={n_cand} P={P} k={k} ties={ties}")
    lg_d = G.dev(lg)
    got = gpu_topk_cand(lg_d, cand, P, rows, 1, k)
    assert np.array_equal(got, gpu_topk_cand(lg_d, cand, P, rows, 1, k)), "deterministic"
    ref = oracle.topk_candidates(lg.astype(np.float64), cand, P, mp, ctx, 1, k)
    for r in range(rows):
        g, o = got[r], ref[r]
        assert np.array_equal(np.sort(g[g >= 0]), np.sort(o[o >= 0])), f"row {r}"
        m = int((o >= 0).sum())
        assert np.all(g[m:] == -1) and np.all(g[:m] >= 0), f"row {r}"


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_candidates_large_pool_sampled_rows(fmt):
    """The 6 GiB pool whose used pages straddle 2 GiB, 4 GiB, 4608 MiB and 4.608e9 B: the
    candidate scorer rebases each page in 64 bits like the dense one."""
    W = wl.make_workload(4, kv_format=fmt)
    strad = set(wl.straddling_pages(max(W.page_stride_bytes, W.page_bytes)))
    seqs = sorted(b for b in range(W.B) if strad & set(W.page_table[b].tolist()))
    G.say(f"candidates large pool fmt={fmt}, sequences {seqs}")
    rng = np.random.default_rng(321 + fmt)
    cand = wl.candidate_blocks(rng, W, 24)
    # the straddling pages' blocks among the candidates of their sequences' rows
    for b in seqs:
        blocks = [i for i, p in enumerate(W.page_table[b].tolist()) if p in strad]
        others = [int(x) for x in cand[b] if x >= 0 and x not in blocks]
        row = sorted(blocks + others[: cand.shape[1] - len(blocks)])
        cand[b] = -1
        cand[b, :len(row)] = row
    rows = np.unique(np.concatenate([seqs, [0, W.B - 1]])).astype(np.int64)
    d = setup_scorer(W, fmt)
    logits = run_cand(W, d, cand)
    ref = check_cand(W, d, cand, logits, rows, f"cand large pool fmt{fmt}")
    got = gpu_topk_cand(logits, cand, W.page_size, W.B, W.n_q, W.topk)[rows]
    check_topk_cand(W, cand, got, ref, rows, W.topk, f"cand topk large pool fmt{fmt}")


def test_candidates_graph_replay_matches_eager():
    """Candidate scorer + candidate top-k captured in a HIP graph: every replay reproduces
    the eager results bit for bit."""
    torch = G.torch_cuda()
    W = wl.make_workload(3)
    cand = G.dev(wl.candidate_blocks(np.random.default_rng(331), W, 12, pad=1))
    d = setup_scorer(W, wl.MXFP4)
    logits = torch.zeros((W.rows, 12 * W.page_size), dtype=torch.float32, device="cuda")
    out = torch.zeros((W.rows, W.topk), dtype=torch.int32, device="cuda")

    def step():
        bd.idx_logits_candidates(d["pool"].view, d["q_d"], d["qs_d"], d["w_d"], d["pt_d"], d["ctx_d"], W.B, W.n_q,
                                 W.H, cand, logits)
        bd.idx_topk_candidates(logits, cand, W.page_size, W.B, W.n_q, W.topk, out)

    G.say("candidates graph replay cfg=3")
    step()
    torch.cuda.synchronize()
    ref_logits, ref_out = logits.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        logits.fill_(5.0)
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits.view(torch.int32), ref_logits.view(torch.int32)), f"replay {rep}: logits"
        assert torch.equal(out, ref_out), f"replay {rep}: top-k"
