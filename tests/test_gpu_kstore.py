"""GPU parity: K-cache store and Q packing are bit-exact against the oracle.

Every used page of the device pool must equal the oracle's bytes; every byte the
store must not touch (gaps between pages, unused pages, slack after a page) must
still hold the canary."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G

pytestmark = pytest.mark.gpu

_cache = {}


def workload(cfg, fmt=wl.MXFP4, **kw):
    key = (cfg, fmt, tuple(sorted(kw.items())))
    if key not in _cache:
        G.say(f"generating workload cfg={cfg} fmt={fmt} {kw}")
        _cache.clear()
        _cache[key] = wl.make_workload(cfg, kv_format=fmt, **kw)
    return _cache[key]


def run_k_store(W, pool, rows=None, pad_every=0):
    torch = G.torch_cuda()
    sel = np.arange(W.k_rows.shape[0]) if rows is None else rows
    slots = W.slots[sel].copy()
    if pad_every:
        slots[::pad_every] = -1
    k = G.bf16_dev(W.k_rows[sel])
    fn = bd.idx_k_store_mxfp4 if pool.fmt == wl.MXFP4 else bd.idx_k_store_fp8
    fn(pool.view, k, G.dev(W.gamma), W.eps, G.dev(W.positions[sel]), G.dev(W.cos_sin), G.dev(slots))
    torch.cuda.synchronize()
    return slots


def test_fp64_division_and_sqrt_are_ieee():
    torch = G.torch_cuda()
    rng = np.random.default_rng(40)
    n = 4_000_000
    a = np.abs(rng.standard_normal(n)) * 10.0 ** rng.integers(-30, 30, n)
    b = rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)
    G.say("diag fp64 n=4e6")
    da, db = G.dev(a), G.dev(b)
    q = torch.empty_like(da)
    r = torch.empty_like(da)
    bd.idx_diag_fp64(da, db, q, r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), a / b)
    np.testing.assert_array_equal(r.cpu().numpy(), np.sqrt(a))


@pytest.mark.parametrize("cfg,fmt,kw", [
    (0, wl.MXFP4, {}),
    (0, wl.FP8, {}),
    (3, wl.MXFP4, {}),
    (3, wl.FP8, {}),
    (2, wl.MXFP4, {"gamma_random": True}),
    (2, wl.FP8, {"gamma_random": True}),
])
def test_k_store_bit_exact(cfg, fmt, kw):
    W = workload(cfg, fmt, **kw)
    G.say(f"k_store cfg={cfg} fmt={fmt} rows={W.k_rows.shape[0]}")
    pool = G.DevicePool(W)
    slots = run_k_store(W, pool, pad_every=7)
    keep = np.where(slots >= 0)[0]
    hp = G.CompactHostPool(W, rows=keep)
    got = pool.read_pages(hp.pids)
    ref = hp.pages()
    np.testing.assert_array_equal(got[:, : hp.page_bytes], ref)
    # slack after each page (stride > page bytes) and pages nobody uses stay canary
    if pool.stride > hp.page_bytes:
        assert np.all(got[:, hp.page_bytes:] == G.CANARY)
    unused = np.setdiff1d(np.arange(W.num_pages), hp.pids)
    if unused.size:
        assert np.all(pool.read_pages(unused[:64]) == G.CANARY)
    if W.offset_bytes:
        assert np.all(pool.base[: W.offset_bytes].cpu().numpy() == G.CANARY)


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_k_store_large_pool_full_size(fmt):
    """The 6 GiB pool with used pages across the 2 GiB / 4 GiB / 4.608 GB boundaries:
    all 2.6M rows stored on the GPU, every used page compared with the oracle."""
    W = workload(4, fmt)
    G.say(f"k_store large pool fmt={fmt} rows={W.k_rows.shape[0]} pool={W.pool_bytes}")
    pool = G.DevicePool(W)
    run_k_store(W, pool)
    hp = G.CompactHostPool(W)
    ref = hp.pages()
    chunk = 4096
    for i in range(0, hp.pids.size, chunk):
        got = pool.read_pages(hp.pids[i: i + chunk])
        np.testing.assert_array_equal(got[:, : hp.page_bytes], ref[i: i + chunk])
    used = set(hp.pids.tolist())
    for pid, boundary in zip(wl.straddling_pages(pool.stride), (1 << 31, 1 << 32, 4608 << 20, 4_608_000_000)):
        assert pid in used and pid * pool.stride < boundary < (pid + 1) * pool.stride


def test_k_store_deterministic_and_idempotent():
    W = workload(3)
    pool = G.DevicePool(W)
    run_k_store(W, pool)
    a = pool.base.clone()
    run_k_store(W, pool)
    G.torch_cuda().cuda.synchronize()
    assert bool((a == pool.base).all())


@pytest.mark.parametrize("fmt", [wl.MXFP4, wl.FP8])
def test_q_quant_bit_exact(fmt):
    torch = G.torch_cuda()
    W = workload(2)
    G.say(f"q_quant fmt={fmt} vecs={W.q_rows.size // 128}")
    q = G.bf16_dev(W.q_rows.reshape(-1, 128))
    n = q.shape[0]
    if fmt == wl.MXFP4:
        qp = torch.empty((n, 64), dtype=torch.uint8, device="cuda")
        qs = torch.empty((n, 4), dtype=torch.uint8, device="cuda")
        bd.idx_q_quant_mxfp4(q, qp, qs)
        rp, rs = oracle.q_quant_mxfp4(W.q_rows.reshape(-1, 128))
        np.testing.assert_array_equal(qp.cpu().numpy(), rp)
        np.testing.assert_array_equal(qs.cpu().numpy(), rs)
    else:
        q8 = torch.empty((n, 128), dtype=torch.uint8, device="cuda")
        wo = torch.empty((n,), dtype=torch.float32, device="cuda")
        bd.idx_q_quant_fp8(q, G.dev(W.w.reshape(-1)), q8, wo)
        r8, rw = oracle.q_quant_fp8(W.q_rows.reshape(-1, 128), W.w.reshape(-1))
        np.testing.assert_array_equal(q8.cpu().numpy(), r8)
        np.testing.assert_array_equal(wo.cpu().numpy().view(np.uint32), rw.view(np.uint32))


def test_k_store_edge_rows():
    """Zero rows, constant rows, a zero row (sign-only codes), huge and tiny values,
    rows at position 0 and at the last table position, and the empty call."""
    torch = G.torch_cuda()
    W = workload(0)
    P = W.page_size
    rows = np.stack([
        wl.f32_to_bf16_bits(np.zeros(128, np.float32)),
        wl.f32_to_bf16_bits(-np.zeros(128, np.float32)),
        wl.f32_to_bf16_bits(np.full(128, 1.0, np.float32)),
        wl.f32_to_bf16_bits(np.full(128, -3.0e38, np.float32)),
        wl.f32_to_bf16_bits(np.full(128, 1.0e-38, np.float32)),
        wl.f32_to_bf16_bits(np.linspace(-5, 5, 128).astype(np.float32)),
    ])
    pos = np.array([0, 3, 0, W.cos_sin.shape[0] - 1, 7, 100], np.int32)
    pids = np.unique(W.page_table[W.page_table >= 0])[:2]
    slots = np.array([pids[0] * P, pids[0] * P + 1, pids[0] * P + P - 1, pids[1] * P, pids[1] * P + 5,
                      pids[1] * P + 63], np.int64)
    for fmt in (wl.MXFP4, wl.FP8):
        pool = G.DevicePool(W, fmt)
        fn = bd.idx_k_store_mxfp4 if fmt == wl.MXFP4 else bd.idx_k_store_fp8
        fn(pool.view, G.bf16_dev(rows), G.dev(W.gamma), W.eps, G.dev(pos), G.dev(W.cos_sin), G.dev(slots))
        fn(pool.view, G.bf16_dev(rows[:0]), G.dev(W.gamma), W.eps, G.dev(pos[:0]), G.dev(W.cos_sin), G.dev(slots[:0]))
        torch.cuda.synchronize()
        page_bytes = wl.BYTES_PER_TOKEN[fmt] * P
        host = np.full(2 * page_bytes, G.CANARY, np.uint8)
        remap = {int(pids[0]): 0, int(pids[1]): 1}
        hslots = np.array([remap[int(s) // P] * P + int(s) % P for s in slots], np.int64)
        oracle.k_store(host, 0, page_bytes, 2, P, fmt, rows, W.gamma, W.eps, pos, W.cos_sin, hslots)
        got = pool.read_pages(pids)[:, :page_bytes].reshape(-1)
        np.testing.assert_array_equal(got, host)
