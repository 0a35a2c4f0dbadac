"""GPU parity: the decode step for callers that cannot allocate (idx_decode_step_noalloc).

Its block counters live in the library's static device array instead of a caller
workspace.  On the same inputs it must give exactly what idx_decode_step gives (the
pool bytes, every logits bit including untouched masked cells, the top-k indices), on
two calls in a row through the C ABI, the second with a smaller input, so that the
array's contents left by one call cannot leak into the next."""
import numpy as np
import pytest

from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G
from tests.test_gpu_step import Step, new_rows

pytestmark = pytest.mark.gpu


def _step_pair(W, fmt):
    ctx = np.asarray(W.ctx, np.int32)
    new = new_rows(W, ctx)
    old = np.setdiff1d(np.arange(W.k_rows.shape[0]), new[new >= 0])
    hp_old = G.CompactHostPool(W, fmt, rows=old)
    return Step(W, fmt, ctx, hp_old), Step(W, fmt, ctx, hp_old)


def _noalloc(s):
    W = s.W
    logits, out = s.buffers()
    bd.idx_decode_step_noalloc(s.pool.view, s.k_d, s.gamma_d, W.eps, s.pos_d, s.cs_d, s.slot_d, s.q_d, s.qs_d, s.w_d,
                               s.pt_d, s.ctx_d, W.B, W.n_q, W.H, W.max_ctx, logits, W.topk, out)
    G.torch_cuda().cuda.synchronize()
    return logits.cpu().numpy(), out.cpu().numpy()


def _check_same(W, fmt, label):
    a, b = _step_pair(W, fmt)
    la, oa = a.fused()        # idx_decode_step with its caller workspace
    lb, ob = _noalloc(b)      # the same step with the library's static counters
    assert np.array_equal(a.pool.read_pages(a.pids), b.pool.read_pages(b.pids)), f"{label}: pool bytes differ"
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), f"{label}: logits bits differ"
    assert np.array_equal(oa, ob), f"{label}: top-k indices differ"
    assert np.all(ob != -5), f"{label}: an output slot was left unwritten"


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_noalloc_matches_workspace_step_twice_shrinking(fmt):
    big = wl.make_workload(1, kv_format=fmt, scale={"B": 24, "ctx": 6000})   # one fused launch, 3 blocks per row
    small = wl.make_workload(0, kv_format=fmt)                                # 2 sequences of 200 / 256 tokens
    assert bd.idx_decode_step_fused(big.B, big.n_q, big.H, big.max_ctx) == 1
    assert bd.idx_decode_step_fused(small.B, small.n_q, small.H, small.max_ctx) == 1
    G.say(f"noalloc step fmt={fmt}: B{big.B}/ctx{big.max_ctx}, then B{small.B}/ctx{small.max_ctx}")
    _check_same(big, fmt, "first call (B24)")
    _check_same(small, fmt, "second call (B2)")


def test_noalloc_rejects_more_sequences_than_its_array():
    W = wl.make_workload(0)
    a, _ = _step_pair(W, wl.MXFP4)
    logits, out = a.buffers()
    B = bd.IDX_NOALLOC_MAX_SEQS + 1
    with pytest.raises(bd.IdxError) as e:
        bd.idx_decode_step_noalloc(a.pool.view, a.k_d, a.gamma_d, W.eps, a.pos_d, a.cs_d, a.slot_d, a.q_d, a.qs_d,
                                   a.w_d, a.pt_d, a.ctx_d, B, W.n_q, W.H, W.max_ctx, logits, W.topk, out)
    assert e.value.status == bd.IDX_ESCRATCH
