"""GPU: page-id guards of every scorer form, and sensitivity controls for the parity checks.

Guards.  The contract says a page id outside the pool is never read: its cells score NaN.
Each form gets a pool whose device allocation holds spare pages past the declared
num_pages and starts at least one page stride before page 0 (a nonzero offset), both
filled with valid-looking K bytes.  The page table then names ids just past the pool and
just below page 0; had a form's guard been missing, it would read those mapped spare bytes
and produce finite logits, never a fault.  Every cell of such a page must be NaN, written
(not the fill sentinel), and the other cells finite.

Sensitivity.  The element-wise comparisons must fail when the GPU's input is corrupted
in bounds: two valid page-table entries swapped, one E8M0 scale byte of a used row
changed, the K store's positions shifted by one (most bytes then differ)."""
import numpy as np
import pytest

from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G
from tests.test_gpu_logits import check, edge_workload, run_scorer, setup_scorer

pytestmark = pytest.mark.gpu

SPARE = 4   # spare pages past num_pages, and pages of offset before page 0


class GuardPool:
    """Random K bytes in a device allocation of SPARE + num_pages + SPARE pages; the view
    starts SPARE pages in and declares num_pages pages."""

    def __init__(self, W, fmt, seed):
        torch = G.torch_cuda()
        rng = np.random.default_rng(seed)
        bpt = wl.BYTES_PER_TOKEN[fmt]
        P = W.page_size
        self.stride = (bpt * P + 255) // 256 * 256
        total_pages = W.num_pages + 2 * SPARE
        host = rng.integers(0, 256, (total_pages, self.stride), dtype=np.uint8)
        if fmt == wl.MXFP4:
            host[:, 64 * P: 68 * P] = rng.integers(120, 131, (total_pages, 4 * P))   # sane E8M0 scales
            host[:, :64 * P] &= 0x77                                               # positive codes
        else:
            codes = rng.integers(0, 0x70, (total_pages, 128 * P)).astype(np.uint8)
            host[:, :128 * P] = codes
            sk = np.full((total_pages, P), 0.01, np.float32)
            host[:, 128 * P: 132 * P] = sk.view(np.uint8).reshape(total_pages, 4 * P)
        self.t = torch.empty((total_pages * self.stride + 256,), dtype=torch.uint8, device="cuda")
        shift = (-self.t.data_ptr()) % 256
        self.base = self.t[shift: shift + total_pages * self.stride]
        self.base.copy_(torch.from_numpy(host.reshape(-1)).to("cuda"))
        self.view = bd.make_pool(self.base, SPARE * self.stride, self.stride, W.num_pages, P, fmt)


def _bad_table(W):
    """The workload's page table with one id just past the pool and one just below page 0
    (both land in the spare pages) in every sequence that has at least two pages."""
    pt = W.page_table.copy()
    bad = []
    for b in range(W.B):
        pages = (int(W.ctx[b]) + W.page_size - 1) // W.page_size
        if pages >= 2:
            pt[b, 0] = W.num_pages + (b % SPARE)          # past the pool
            pt[b, pages - 1] = -1 - (b % SPARE)           # below page 0
            bad.append((b, 0))
            bad.append((b, pages - 1))
    assert bad
    return pt, bad


def _scores(W, fmt, form):
    torch = G.torch_cuda()
    gp = GuardPool(W, fmt, seed=W.H * 7 + W.n_q)
    q, qs, w = G.oracle_q(W, fmt)
    pt, bad = _bad_table(W)
    logits = torch.empty((W.rows, W.max_ctx + 3), dtype=torch.float32, device="cuda")
    logits.view(torch.int32).fill_(np.int32(np.uint32(G.SENTINEL_BITS).view(np.int32)))
    args = (gp.view, G.dev(q), None if qs is None else G.dev(qs), G.dev(w), G.dev(pt), G.dev(W.ctx), W.B, W.n_q, W.H)
    if form == "candidates":
        cand = np.tile(np.arange(pt.shape[1], dtype=np.int32), (W.rows, 1))   # every block of the row, in order
        logits = torch.empty((W.rows, cand.shape[1] * W.page_size), dtype=torch.float32, device="cuda")
        bd.idx_logits_candidates(*args, G.dev(cand), logits)
    elif form == "step":
        new = np.full(W.rows, -1, np.int64)              # no new rows: the step scores the pool as it is
        k_new = G.bf16_dev(np.zeros((W.rows, 128), np.uint16))
        out = torch.empty((W.rows, W.topk), dtype=torch.int32, device="cuda")
        ws = torch.zeros(bd.idx_workspace_bytes(W.B, W.n_q, W.H, W.max_ctx, W.topk) // 4, dtype=torch.int32,
                         device="cuda")
        assert bd.idx_decode_step_fused(W.B, W.n_q, W.H, W.max_ctx) == 1
        bd.idx_decode_step(gp.view, k_new, G.dev(np.ones(128, np.float32)), 1e-6, G.dev(np.zeros(W.rows, np.int32)),
                           G.dev(W.cos_sin), G.dev(new), *args[1:], W.max_ctx, logits, W.topk, out, ws)
    else:
        bd.idx_logits_paged(*args, W.max_ctx, logits)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), bad


@pytest.mark.parametrize("form,H,n_q,P,ctx,fmt", [
    ("decode", 4, 1, 64, [200, 256], wl.MXFP4),              # one-pass decode form
    ("decode", 32, 1, 128, [700, 1300, 260], wl.FP8),
    ("prefill", 32, 33, 128, [40, 1000], wl.MXFP4),           # prefill form
    ("stream", 64, 3, 64, [300, 900, 2368, 130], wl.MXFP4),   # balanced streaming form, several rows
    ("stream", 64, 3, 64, [500, 1200], wl.FP8),
    ("rows", 16, 9, 64, [200, 700], wl.MXFP4),                # row-split decode form
    ("candidates", 32, 1, 64, [400, 1000], wl.MXFP4),         # candidate-block scorer
    ("step", 32, 1, 128, [1000, 3000], wl.MXFP4),             # fused decode step
])
def test_page_id_outside_the_pool_scores_nan(form, H, n_q, P, ctx, fmt):
    W = edge_workload(H, n_q, P, ctx, fmt)
    G.say(f"guards form={form} H={H} n_q={n_q} P={P} ctx={ctx} fmt={fmt}")
    got, bad = _scores(W, fmt, form)
    bits = got.view(np.uint32)
    badset = set(bad)
    for r in range(W.rows):
        b = r // W.n_q
        n = W.valid_len(r)
        for p in range((n + P - 1) // P):
            lo, hi = p * P, min((p + 1) * P, n)
            # (candidates: every block of the row in order, so cell c*P + i is token c*P + i)
            cells, cbits = got[r, lo:hi], bits[r, lo:hi]
            if (b, p) in badset:
                assert np.all(np.isnan(cells)) and np.all(cbits != G.SENTINEL_BITS), \
                    f"{form}: row {r} page {p} outside the pool did not score NaN"
            else:
                assert np.all(np.isfinite(cells)), f"{form}: row {r} page {p} not finite"


# ------------------------------------------------------------------------ sensitivity
def _raises_parity(fn):
    with pytest.raises(AssertionError):
        fn()


def test_parity_check_fails_on_swapped_page_table_entries():
    W = wl.make_workload(0)
    d = setup_scorer(W, wl.MXFP4)
    logits = run_scorer(W, d)
    check(W, d, logits, np.arange(W.rows), "control: unchanged")      # passes
    pt = W.page_table.copy()
    pt[0, 0], pt[0, 1] = pt[0, 1], pt[0, 0]                            # both valid: an in-bounds corruption
    d2 = dict(d, pt_d=G.dev(pt))
    bad = run_scorer(W, d2)
    _raises_parity(lambda: check(W, d, bad, np.arange(W.rows), "control: swapped pages"))


def test_parity_check_fails_on_changed_scale_bytes():
    W = wl.make_workload(0)
    d = setup_scorer(W, wl.MXFP4)
    pool = d["pool"]
    pid = int(W.page_table[1, 2])                    # tokens 128..191 of sequence 1 (256 valid)
    for row in range(16):
        off = pool.offset + pid * pool.stride + 64 * W.page_size + 4 * row + 1   # block 1 of the token
        pool.base[off: off + 1].add_(3)                                          # that block's scale x 8
    bad = run_scorer(W, d)
    _raises_parity(lambda: check(W, d, bad, np.arange(W.rows), "control: one scale byte"))


def test_k_store_bytes_change_with_shifted_positions():
    """The K store's bit-exact check has teeth: positions shifted by one (every row rotated
    by the wrong angle) change most stored bytes against the oracle's."""
    torch = G.torch_cuda()
    W = wl.make_workload(0)
    hp = G.CompactHostPool(W, wl.MXFP4)
    pool = G.DevicePool(W, wl.MXFP4)
    pos = np.minimum(W.positions + 1, W.cos_sin.shape[0] - 1).astype(np.int32)
    bd.idx_k_store_mxfp4(pool.view, G.bf16_dev(W.k_rows), G.dev(W.gamma), W.eps, G.dev(pos), G.dev(W.cos_sin),
                         G.dev(W.slots))
    torch.cuda.synchronize()
    got = pool.read_pages(hp.pids)[:, : hp.page_bytes]
    ref = hp.pages()
    assert not np.array_equal(got, ref)
    # over the stored rows' own bytes: the 32 nibble bytes of the rotated dims 0..63 and the
    # two scale bytes of their blocks (dims 64..127 are not rotated, so they match)
    P = W.page_size
    page_of = {int(p): i for i, p in enumerate(hp.pids)}
    diff = []
    for slot in W.slots:
        i, row = page_of[int(slot) // P], int(slot) % P
        g = np.concatenate([got[i, 64 * row: 64 * row + 32], got[i, 64 * P + 4 * row: 64 * P + 4 * row + 2]])
        rr = np.concatenate([ref[i, 64 * row: 64 * row + 32], ref[i, 64 * P + 4 * row: 64 * P + 4 * row + 2]])
        diff.append(np.mean(g != rr))
    frac = float(np.mean(diff))
    G.say(f"shifted positions: {frac:.3f} of the rotated dims' bytes differ")
    assert frac > 0.2
