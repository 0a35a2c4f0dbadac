"""GPU parity: the fused decode step (idx_decode_step).

The pool starts with the oracle's bytes of every cached row except the step's new rows
(the newest n_q tokens of each sequence), whose slots hold the canary.  Then:
  - against the separate entry points on the same inputs (idx_k_store_*, then
    idx_logits_paged, then idx_topk): the pool bytes, the logits bits of every valid
    cell and the top-k index arrays are identical;
  - against the oracle: the pool bytes equal the oracle's K store of every row, the
    logits meet the scorer's tolerance and the top-k meets the tolerance rule;
  - the workspace is zero again after each call, and a repeated call gives the same
    bytes."""
import numpy as np
import pytest

from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def new_rows(W, ctx):
    """K-row indices of the step's new tokens: row b*n_q + j of the step is token
    ctx[b] - n_q + j of sequence b (-1 where that index is negative)."""
    out = []
    for o, c in zip(W.seq_row_offsets()[:-1], ctx):
        for j in range(W.n_q):
            t = int(c) - W.n_q + j
            out.append(int(o) + t if t >= 0 else -1)
    return np.array(out, np.int64)


class Step:
    """Device inputs of one decode step of workload W (pool without the new rows)."""

    def __init__(self, W, fmt, ctx, hp_old):
        torch = G.torch_cuda()
        self.W, self.fmt = W, fmt
        self.ctx = np.asarray(ctx, np.int32)
        self.new = new_rows(W, self.ctx)
        have = self.new >= 0
        self.pool = G.DevicePool(W, fmt)
        self.pool.write_pages(hp_old.pids, hp_old.pages())
        self.pids = hp_old.pids
        q, qs, w = G.oracle_q(W, fmt)
        self.q, self.qs, self.w = q, qs, w
        self.q_d, self.qs_d, self.w_d = G.dev(q), None if qs is None else G.dev(qs), G.dev(w)
        self.pt_d, self.ctx_d = G.dev(W.page_table), G.dev(self.ctx)
        src = np.where(have, self.new, 0)
        k_new = W.k_rows[src]
        self.k_d = G.bf16_dev(k_new)
        self.pos_d = G.dev(np.where(have, W.positions[src], 0).astype(np.int32))
        self.slot_np = np.where(have, W.slots[src], -1).astype(np.int64)
        self.slot_d = G.dev(self.slot_np)
        self.gamma_d, self.cs_d = G.dev(W.gamma), G.dev(W.cos_sin)
        self.ws = torch.zeros(bd.idx_workspace_bytes(W.B, W.n_q, W.H, W.max_ctx, W.topk) // 4, dtype=torch.int32,
                              device="cuda")

    def buffers(self):
        torch = G.torch_cuda()
        W = self.W
        logits = torch.empty((W.rows, W.max_ctx), dtype=torch.float32, device="cuda")
        logits.view(torch.int32).fill_(np.int32(np.uint32(G.SENTINEL_BITS).view(np.int32)))
        out = torch.full((W.rows, W.topk), -5, dtype=torch.int32, device="cuda")
        return logits, out

    def fused(self):
        W = self.W
        logits, out = self.buffers()
        bd.idx_decode_step(self.pool.view, self.k_d, self.gamma_d, W.eps, self.pos_d, self.cs_d, self.slot_d,
                           self.q_d, self.qs_d, self.w_d, self.pt_d, self.ctx_d, W.B, W.n_q, W.H, W.max_ctx, logits,
                           W.topk, out, self.ws)
        G.torch_cuda().cuda.synchronize()
        return logits.cpu().numpy(), out.cpu().numpy()

    def separate(self):
        W = self.W
        logits, out = self.buffers()
        store = bd.idx_k_store_mxfp4 if self.fmt == wl.MXFP4 else bd.idx_k_store_fp8
        store(self.pool.view, self.k_d, self.gamma_d, W.eps, self.pos_d, self.cs_d, self.slot_d)
        bd.idx_logits_paged(self.pool.view, self.q_d, self.qs_d, self.w_d, self.pt_d, self.ctx_d, W.B, W.n_q, W.H,
                            W.max_ctx, logits)
        bd.idx_topk(logits, self.ctx_d, W.B, W.n_q, W.topk, out)
        G.torch_cuda().cuda.synchronize()
        return logits.cpu().numpy(), out.cpu().numpy()


def valid_cells(W, ctx):
    n = np.array([max(0, min(int(ctx[r // W.n_q]) - W.n_q + 1 + r % W.n_q, int(ctx[r // W.n_q])))
                  for r in range(W.rows)])
    return np.arange(W.max_ctx)[None, :] < n[:, None]


def compare_paths(W, fmt, ctx=None, slot_override=None, label=""):
    ctx = np.asarray(W.ctx if ctx is None else ctx, np.int32)
    new = new_rows(W, ctx)
    old = np.setdiff1d(np.arange(W.k_rows.shape[0]), new[new >= 0])
    hp_old = G.CompactHostPool(W, fmt, rows=old)  # every cached row but the step's new ones
    a, b = Step(W, fmt, ctx, hp_old), Step(W, fmt, ctx, hp_old)
    for s in (a, b):
        if slot_override is not None:
            s.slot_np = slot_override(s.slot_np.copy())
            s.slot_d = G.dev(s.slot_np)
    la, oa = a.separate()
    lb, ob = b.fused()
    pa, pb = a.pool.read_pages(a.pids), b.pool.read_pages(b.pids)
    assert np.array_equal(pa, pb), f"{label}: pool bytes differ from the separate K store"
    mask = valid_cells(W, a.ctx)
    assert np.array_equal(la.view(np.uint32)[mask], lb.view(np.uint32)[mask]), f"{label}: logits bits differ"
    assert np.all(lb.view(np.uint32)[~mask] == G.SENTINEL_BITS), f"{label}: a masked cell was written"
    assert np.array_equal(oa, ob), f"{label}: top-k indices differ"
    assert int(b.ws.abs().sum().item()) == 0, f"{label}: workspace not left zero"
    lb2, ob2 = b.fused()
    assert np.array_equal(lb.view(np.uint32), lb2.view(np.uint32)) and np.array_equal(ob, ob2), f"{label}: repeat"
    assert int(b.ws.abs().sum().item()) == 0
    return b, lb, ob


@pytest.mark.parametrize("cfg,fmt", [(0, wl.MXFP4), (0, wl.FP8), (1, wl.MXFP4), (1, wl.FP8)])
def test_step_matches_separate_calls_and_oracle(cfg, fmt):
    W = wl.make_workload(cfg, kv_format=fmt)
    G.say(f"decode step cfg={cfg} fmt={fmt}")
    st, logits, out = compare_paths(W, fmt, label=f"cfg{cfg}/fmt{fmt}")
    hp = G.CompactHostPool(W, fmt)  # the oracle's K store of every row
    assert np.array_equal(st.pool.read_pages(hp.pids)[:, :hp.page_bytes], hp.pages()), "pool bytes vs oracle"
    rows = np.arange(W.rows)
    ref = G.oracle_logits(hp, st.q, st.qs, st.w, rows, W.max_ctx)
    mask = G.valid_mask(W, rows, W.max_ctx)
    stats = G.assert_logits_close(logits, ref, mask, f"cfg{cfg}/fmt{fmt}")
    G.assert_topk_valid(out, ref, W, rows, W.topk, 1e-4 * stats["max_abs_ref"], f"cfg{cfg}/fmt{fmt}")
    G.say(f"cfg{cfg}/fmt{fmt}: {stats}")


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_step_large_pool(fmt):
    """B256, contexts up to 16384 in a 6 GiB pool: identical to the separate calls; the
    oracle checks sampled rows."""
    W = wl.make_workload(4, kv_format=fmt)
    G.say(f"decode step large pool fmt={fmt}")
    st, logits, out = compare_paths(W, fmt, label=f"cfg4/fmt{fmt}")
    rows = np.array([0, 17, 100, 255])
    hp = G.CompactHostPool(W, fmt)
    ref = G.oracle_logits(hp, st.q, st.qs, st.w, rows, W.max_ctx)
    mask = G.valid_mask(W, rows, W.max_ctx)
    stats = G.assert_logits_close(logits[rows], ref, mask, f"cfg4/fmt{fmt}")
    G.assert_topk_valid(out[rows], ref, W, rows, W.topk, 1e-4 * stats["max_abs_ref"], f"cfg4/fmt{fmt}")


@pytest.mark.parametrize("cfg,fmt,scale", [
    (1, wl.MXFP4, {"B": 16, "H": 64}),            # 64 heads of one query token: four head tiles
    (1, wl.FP8, {"B": 6, "H": 64}),
    (3, wl.MXFP4, {"B": 8, "H": 16}),             # three query tokens of 16 heads, page 64, offset pool
    (3, wl.MXFP4, {"B": 10}),                     # three query tokens of 64 heads: the streaming scorer
    (1, wl.MXFP4, {"B": 12, "H": 32, "n_q": 2}),  # two query tokens of 32 heads
])
def test_step_more_head_tiles(cfg, fmt, scale):
    """Shapes with more query head tiles than the fused kernel holds run as the three
    kernels inside the entry point: the same bytes and bits as the separate calls, and
    the oracle within the tolerances."""
    W = wl.make_workload(cfg, kv_format=fmt, scale=scale)
    G.say(f"decode step cfg={cfg} fmt={fmt} {scale} (n_q={W.n_q}, H={W.H})")
    b, lb, ob = compare_paths(W, fmt, label=f"cfg{cfg}/{scale}")
    rows = np.arange(W.rows)
    hp = G.CompactHostPool(W, fmt)
    ref = G.oracle_logits(hp, b.q, b.qs, b.w, rows, W.max_ctx)
    mask = G.valid_mask(W, rows, W.max_ctx)
    stats = G.assert_logits_close(lb, ref, mask, f"cfg{cfg}/{scale}")
    G.assert_topk_valid(ob, ref, W, rows, W.topk, 1e-4 * stats["max_abs_ref"], f"cfg{cfg}/{scale}")


def test_step_fused_query():
    """Which shapes run as the one fused kernel (on a device with at least 256 CUs)."""
    assert bd.idx_decode_step_fused(64, 1, 32, 8192) == 1      # decode B64/H32/8K: 256 blocks
    assert bd.idx_decode_step_fused(2, 1, 4, 256) == 1
    assert bd.idx_decode_step_fused(256, 1, 32, 16384) == 0    # more blocks than CUs
    assert bd.idx_decode_step_fused(16, 1, 64, 8192) == 0      # four head tiles
    assert bd.idx_decode_step_fused(4, 1, 32, 20000) == 0      # rows past the fused top-k's
    assert bd.idx_decode_step_fused(4, 1, 32, 0) == 0


def test_step_rejects_prefill_shapes():
    """More than 16 query head tiles per sequence is the scorer's prefill form, which the
    decode step does not take: IDX_EUNSUPPORTED before anything is enqueued."""
    W = wl.make_workload(1, scale={"B": 2, "H": 64, "n_q": 5, "ctx": 512})
    ctx = np.asarray(W.ctx, np.int32)
    new = new_rows(W, ctx)
    old = np.setdiff1d(np.arange(W.k_rows.shape[0]), new[new >= 0])
    st = Step(W, wl.MXFP4, ctx, G.CompactHostPool(W, wl.MXFP4, rows=old))
    logits, out = st.buffers()
    with pytest.raises(bd.IdxError) as e:
        bd.idx_decode_step(st.pool.view, st.k_d, st.gamma_d, W.eps, st.pos_d, st.cs_d, st.slot_d, st.q_d, st.qs_d,
                           st.w_d, st.pt_d, st.ctx_d, W.B, W.n_q, W.H, W.max_ctx, logits, W.topk, out, st.ws)
    assert e.value.status == bd.IDX_EUNSUPPORTED


def test_step_edges():
    """A padding slot (the row is neither stored nor substituted), an empty sequence and
    a sequence of one token, a context that is not a multiple of the block's tokens."""
    W = wl.make_workload(1, scale={"B": 6})
    G.say("decode step edges")
    ctx = W.ctx.copy()
    ctx[1] = 0
    ctx[2] = 1
    ctx[3] = 3001
    def pad(sl):
        sl[4] = -1
        return sl
    compare_paths(W, wl.MXFP4, ctx=ctx, slot_override=pad, label="edges")


@pytest.mark.parametrize("cfg,scale", [(1, {"B": 16}), (4, {"B": 24})])
def test_step_xcd_grouped_mixed_lengths(cfg, scale):
    """B a multiple of the XCD count, so the fused kernel places a sequence's blocks on one
    XCD (its grouped block order), with mixed lengths down to one token, so sequences end
    in different chunks and some chunks are empty: 16 sequences of up to 8192 tokens (4
    chunks), 24 of up to 16384 (8 chunks, 192 blocks)."""
    W = wl.make_workload(cfg, scale=scale)
    assert W.B % 8 == 0 and bd.idx_decode_step_fused(W.B, W.n_q, W.H, W.max_ctx) == 1
    rng = np.random.default_rng(70 + W.B)
    ctx = np.array([rng.integers(1, int(c) + 1) for c in W.ctx], np.int32)
    ctx[0], ctx[-1] = 1, W.ctx[-1]
    G.say(f"decode step, grouped block order, cfg={cfg} B={W.B}")
    compare_paths(W, wl.MXFP4, ctx=ctx, label=f"grouped cfg{cfg} B{W.B}")


@pytest.mark.parametrize("cfg,scale", [(1, {"B": 6}), (4, {"B": 40})])
def test_step_skips_rows_before_the_first_token(cfg, scale):
    """A row whose token index ctx[b] - n_q + j is negative is not stored even with a
    valid slot — in the fused kernel (6 sequences) and in the three-kernel sequence the
    entry point runs when the grid exceeds one block per CU (40 sequences of up to 16384
    tokens)."""
    W = wl.make_workload(cfg, scale=scale)
    G.say(f"decode step, empty sequence with a valid slot, cfg={cfg} B={W.B}")
    ctx = W.ctx.copy()
    ctx[1] = 0
    new = new_rows(W, ctx)
    old = np.setdiff1d(np.arange(W.k_rows.shape[0]), new[new >= 0])
    hp_old = G.CompactHostPool(W, wl.MXFP4, rows=old)
    st = Step(W, wl.MXFP4, ctx, hp_old)
    pid = int(W.page_table[1][0])
    st.slot_np[1] = pid * W.page_size + 5   # the slot of token 5 of sequence 1
    st.slot_d = G.dev(st.slot_np)
    before = st.pool.read_pages(np.array([pid]))
    logits, out = st.fused()
    after = st.pool.read_pages(np.array([pid]))
    assert np.array_equal(before, after), "a row with a negative token index was stored"
    assert np.all(out[1] == -1), "the empty sequence's row must be all -1"


def test_step_graph_replay_matches_eager():
    """The fused step captured in a HIP graph: every replay (eager work and a sync between
    replays) reproduces the eager call's pool bytes, logits bits and indices, and leaves the
    workspace zero (the kernel resets its own counters, so no memset node is needed)."""
    torch = G.torch_cuda()
    W = wl.make_workload(1)
    ctx = np.asarray(W.ctx, np.int32)
    new = new_rows(W, ctx)
    old = np.setdiff1d(np.arange(W.k_rows.shape[0]), new[new >= 0])
    st = Step(W, wl.MXFP4, ctx, G.CompactHostPool(W, wl.MXFP4, rows=old))
    logits, out = st.buffers()

    def step():
        bd.idx_decode_step(st.pool.view, st.k_d, st.gamma_d, W.eps, st.pos_d, st.cs_d, st.slot_d, st.q_d, st.qs_d,
                           st.w_d, st.pt_d, st.ctx_d, W.B, W.n_q, W.H, W.max_ctx, logits, W.topk, out, st.ws)

    G.say("fused step graph replay cfg=1")
    step()
    torch.cuda.synchronize()
    ref_pool, ref_logits, ref_out = st.pool.base.clone(), logits.clone(), out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        logits.copy_(ref_logits)
        logits[:, :64].fill_(3.0)   # cells every row rewrites
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bool((st.pool.base == ref_pool).all()), f"replay {rep}: pool"
        assert torch.equal(logits.view(torch.int32), ref_logits.view(torch.int32)), f"replay {rep}: logits"
        assert torch.equal(out, ref_out), f"replay {rep}: top-k"
        assert int(st.ws.abs().sum().item()) == 0, f"replay {rep}: workspace"
