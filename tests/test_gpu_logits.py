"""GPU parity: the paged MQA scorer against the oracle.

K cache bytes and packed Q come from the oracle; the HIP scorer and the oracle read
the same bytes.  Logits must meet max|d| <= 1e-4 * max|ref| and cosine >= 0.999999
over the valid cells of each call; masked cells must keep the sentinel the buffer was
filled with.  Full-size configurations are compared on sampled rows (all rows where
the oracle finishes in seconds), always in the launch configuration of the full call."""
import numpy as np
import pytest

from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def setup_scorer(W, fmt, rows_for_k=None):
    """Device pool filled with the oracle's K bytes, oracle-packed Q, device tensors."""
    hp = G.CompactHostPool(W, fmt, rows=rows_for_k)
    pool = G.DevicePool(W, fmt)
    pool.write_pages(hp.pids, hp.pages())
    q, qs, w = G.oracle_q(W, fmt)
    d = dict(pool=pool, hp=hp, q=q, qs=qs, w=w, q_d=G.dev(q), qs_d=None if qs is None else G.dev(qs), w_d=G.dev(w),
             pt_d=G.dev(W.page_table), ctx_d=G.dev(W.ctx))
    return d


def run_scorer(W, d, stride=None):
    torch = G.torch_cuda()
    stride = stride or W.max_ctx
    logits = torch.empty((W.rows, stride), dtype=torch.float32, device="cuda")
    logits.view(torch.int32).fill_(np.int32(np.uint32(G.SENTINEL_BITS).view(np.int32)))
    bd.idx_logits_paged(d["pool"].view, d["q_d"], d["qs_d"], d["w_d"], d["pt_d"], d["ctx_d"], W.B, W.n_q, W.H,
                        W.max_ctx, logits)
    torch.cuda.synchronize()
    return logits


def check(W, d, logits, rows, label):
    got = logits.cpu().numpy()[rows]
    ref = G.oracle_logits(d["hp"], d["q"], d["qs"], d["w"], rows, got.shape[1])
    mask = G.valid_mask(W, rows, got.shape[1])
    stats = G.assert_logits_close(got, ref, mask, label)
    bits = got.view(np.uint32)
    assert np.all(bits[~mask] == G.SENTINEL_BITS), f"{label}: a masked cell was written"
    G.say(f"{label}: {stats}")
    return got, ref, stats


@pytest.mark.parametrize("cfg,fmt", [(0, wl.MXFP4), (0, wl.FP8), (1, wl.MXFP4), (3, wl.MXFP4), (3, wl.FP8)])
def test_logits_all_rows(cfg, fmt):
    W = wl.make_workload(cfg, kv_format=fmt)
    G.say(f"logits cfg={cfg} fmt={fmt} rows={W.rows}")
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d)
    check(W, d, logits, np.arange(W.rows), f"cfg{cfg}/fmt{fmt}")


def test_logits_prefill_sampled_rows():
    W = wl.make_workload(2)
    G.say("logits prefill cfg=2 (8192 causal rows), sampled")
    d = setup_scorer(W, wl.MXFP4)
    logits = run_scorer(W, d)
    rng = np.random.default_rng(50)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 17, 1023, 1024, 1025, 4095, 8190, 8191],
                                     rng.integers(0, W.rows, 40)]))
    check(W, d, logits, rows, "cfg2 sampled")


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_logits_large_pool_sampled_rows(fmt):
    W = wl.make_workload(4, kv_format=fmt)
    G.say(f"logits large pool fmt={fmt}, sampled")
    # sequences holding the pages that straddle the address boundaries, plus random ones
    strad = set(wl.straddling_pages(max(W.page_stride_bytes, W.page_bytes)))
    seqs = [b for b in range(W.B) if strad & set(W.page_table[b].tolist())]
    rng = np.random.default_rng(51)
    seqs = np.unique(np.concatenate([seqs, rng.integers(0, W.B, 6), [0, W.B - 1]])).astype(np.int64)
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d)
    check(W, d, logits, seqs, f"cfg4/fmt{fmt}")


def edge_workload(H, n_q, P, ctx, fmt=wl.MXFP4):
    rng = np.random.default_rng(H * 1000 + n_q)
    ctx = np.array(ctx, np.int32)
    B = ctx.size
    need = [max((int(c) + P - 1) // P, 0) for c in ctx]
    num_pages = max(sum(need), 1) + 5
    perm = rng.permutation(num_pages)
    pt = np.full((B, max(max(need), 1)), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[pos:pos + n]
        pos += n
    seq = np.repeat(np.arange(B, dtype=np.int32), ctx)
    posn = np.concatenate([np.arange(int(c), dtype=np.int32) for c in ctx]) if ctx.sum() else np.zeros(0, np.int32)
    slots = pt[seq, posn // P].astype(np.int64) * P + posn % P
    bpt = 68 if fmt == wl.MXFP4 else 132
    W = wl.Workload(name="edge", B=B, n_q=n_q, H=H, page_size=P, topk=8, kv_format=fmt, ctx=ctx,
                    num_pages=num_pages, offset_bytes=512, page_stride_bytes=(bpt * P + 256 + 255) // 256 * 256,
                    page_table=pt,
                    k_rows=wl.f32_to_bf16_bits(rng.standard_normal((int(ctx.sum()), 128), dtype=np.float32)),
                    k_seq=seq, positions=posn, slots=slots,
                    q_rows=wl.f32_to_bf16_bits(rng.standard_normal((B, n_q, H, 128), dtype=np.float32)),
                    w=(rng.standard_normal((B, n_q, H)) / np.sqrt(H)).astype(np.float32),
                    gamma=np.ones(128, np.float32), eps=1e-6, cos_sin=wl.rope_cos_sin(max(int(ctx.max()), 1)),
                    seed=0)
    return W


@pytest.mark.parametrize("H,n_q,P,ctx,fmt", [
    (1, 1, 16, [1, 17, 300], wl.MXFP4),        # single head, tiny pages
    (20, 2, 32, [0, 5, 100], wl.MXFP4),        # ragged head tile, empty sequence, n_q > ctx
    (48, 1, 256, [700, 513], wl.MXFP4),        # 3 head tiles, large pages
    (128, 1, 64, [129, 64], wl.MXFP4),         # the largest head count
    (16, 9, 64, [200, 9, 3], wl.MXFP4),        # nine rows of one head tile: the row-split decode kernel
    (48, 5, 64, [300, 70, 5], wl.MXFP4),       # row-split decode kernel, three head tiles per row
    (48, 5, 64, [300, 70, 5], wl.FP8),         # the same in FP8
    (32, 8, 128, [900, 260], wl.FP8),          # row-split decode kernel, two head tiles, FP8, 16 tiles in all
    (32, 33, 128, [40, 1000], wl.MXFP4),       # prefill kernel, causal rows crossing chunk edges
    (32, 33, 128, [40, 1000], wl.FP8),         # the same in FP8
    (20, 17, 64, [17, 700, 0], wl.FP8),        # FP8 prefill, ragged head tile, an empty sequence
    (128, 5, 64, [300], wl.MXFP4),             # prefill form with 8 head tiles
    (16, 40, 64, [2500, 50], wl.MXFP4),        # prefill, one head tile, rows crossing the 1024-token chunks
    (48, 24, 32, [2100, 700], wl.MXFP4),       # prefill, three head tiles, 32-token pages
    (32, 40, 128, [2500, 1030], wl.FP8),       # FP8 prefill across chunk edges
])
def test_logits_shapes_and_edges(H, n_q, P, ctx, fmt):
    W = edge_workload(H, n_q, P, ctx, fmt)
    G.say(f"logits edge H={H} n_q={n_q} P={P} ctx={list(ctx)} fmt={fmt}")
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d, stride=max(W.max_ctx, 1) + 3)
    check(W, d, logits, np.arange(W.rows), f"edge H{H} nq{n_q} P{P} fmt{fmt}")


def test_bad_page_id_scores_nan_without_faulting():
    torch = G.torch_cuda()
    W = wl.make_workload(0)
    d = setup_scorer(W, wl.MXFP4)
    pt = W.page_table.copy()
    pt[1, 1] = W.num_pages + 1000     # outside the pool
    pt[0, 0] = -7
    d["pt_d"] = G.dev(pt)
    logits = run_scorer(W, d)
    got = logits.cpu().numpy()
    P = W.page_size
    bits = got.view(np.uint32)
    for cells in (got[1, P: 2 * P], got[0, :P]):
        assert np.all(np.isnan(cells))
    # NaN was written (not the fill sentinel left untouched)
    assert np.all(bits[1, P: 2 * P] != G.SENTINEL_BITS) and np.all(bits[0, :P] != G.SENTINEL_BITS)
    good = np.isfinite(got[0, P:200])
    assert good.all()
    torch.cuda.synchronize()


def test_scorer_deterministic():
    W = wl.make_workload(3)
    d = setup_scorer(W, wl.MXFP4)
    a = run_scorer(W, d).cpu().numpy()
    b = run_scorer(W, d).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("scale", [
    {"B": 12, "n_q": 2, "H": 48},            # two rows: two waves score, all four fetch K
    {"B": 8, "n_q": 4, "H": 32},             # four rows: every wave scores
    {"B": 9, "n_q": 3, "H": 64, "ctx": 300}, # short contexts: one or two chunks per row
])
@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_logits_streaming_shapes(scale, fmt):
    """The streaming scorer for 2-4 query rows with more than four head tiles in all (K
    shared through LDS by the block's row waves, balanced runs of chunks) on mixed context
    lengths, page 64, an offset pool with gaps: every row against the oracle, masked cells
    untouched."""
    W = wl.make_workload(3, kv_format=fmt, scale=scale)
    G.say(f"logits streaming form fmt={fmt} {scale}")
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d)
    check(W, d, logits, np.arange(W.rows), f"stream {scale}/fmt{fmt}")


def test_logits_streaming_long_runs_small_pages():
    """One-row streaming form with 16-token pages and runs of about a dozen 64-token chunks
    (about 50 pages per run, read from the run's page-id window): every row against the
    oracle.  1.55M tokens over four sequences, so that the streaming form takes the call."""
    W = edge_workload(4, 1, 16, [600_000, 550_000, 300_000, 100_000])
    G.say("logits streaming form, long runs over 16-token pages")
    d = setup_scorer(W, wl.MXFP4)
    logits = run_scorer(W, d)
    check(W, d, logits, np.arange(W.rows), "stream long runs P16")


@pytest.mark.parametrize("n_q,fmt", [(3, wl.MXFP4), (2, wl.FP8)])
def test_logits_streaming_many_sequences(n_q, fmt):
    """150 sequences of mixed lengths (three per lane in the device-side prefix that sizes
    the balanced runs), some empty or shorter than n_q: every row against the oracle."""
    rng = np.random.default_rng(90 + n_q)
    ctx = rng.integers(0, 1500, 150)
    ctx[::17] = 0
    ctx[5::23] = 1
    W = edge_workload(64, n_q, 64, ctx.tolist(), fmt)
    G.say(f"logits streaming form, 150 sequences n_q={n_q} fmt={fmt}")
    d = setup_scorer(W, fmt)
    logits = run_scorer(W, d, stride=W.max_ctx + 3)
    check(W, d, logits, np.arange(W.rows), f"stream 150 seqs nq{n_q}/fmt{fmt}")


@pytest.mark.parametrize("form,H,n_q,P,ctx,fmt", [
    ("prefill", 32, 40, 128, [2500, 1030], wl.MXFP4),
    ("stream", 32, 1, 128, [140000, 100, 3000, 64, 1, 0, 5000, 77, 9, 650, 2048, 64, 63, 65, 1000, 17], wl.MXFP4),
    ("stream", 32, 1, 128, [140000, 100, 3000, 64, 1, 0, 5000, 77, 9, 650, 2048, 64, 63, 65, 1000, 17], wl.FP8),
])
def test_scorer_graph_replay_matches_eager(form, H, n_q, P, ctx, fmt):
    """The prefill form (its unit table built on the host at capture) and the one-row
    streaming form (its runs computed on the device from the lengths) captured in a HIP
    graph: every replay, with eager work and a synchronisation between replays, writes the
    eager call's logits bit for bit."""
    torch = G.torch_cuda()
    W = edge_workload(H, n_q, P, ctx, fmt)
    G.say(f"scorer graph replay form={form} fmt={fmt}")
    d = setup_scorer(W, fmt)
    sentinel = np.int32(np.uint32(G.SENTINEL_BITS).view(np.int32))
    logits = torch.empty((W.rows, W.max_ctx + 3), dtype=torch.float32, device="cuda")

    def call():
        bd.idx_logits_paged(d["pool"].view, d["q_d"], d["qs_d"], d["w_d"], d["pt_d"], d["ctx_d"], W.B, W.n_q, W.H,
                            W.max_ctx, logits)

    logits.view(torch.int32).fill_(sentinel)
    call()
    torch.cuda.synchronize()
    ref = logits.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        logits.view(torch.int32).fill_(sentinel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
    if form == "stream":  # and every row against the oracle (this shape is not covered elsewhere)
        check(W, d, logits, np.arange(W.rows), f"graph {form}/fmt{fmt}")
