"""Shared set-up for the GPU parity tests: device pools, oracle-side compact pools and
the comparison rules.  Inputs come from the seeded generators or from the oracle;
nothing the HIP path produces is ever fed to the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl

CANARY = 0xA5
SENTINEL_BITS = 0x7FC0DEAD  # a NaN payload the kernels never produce


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev(a: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def bf16_dev(bits: np.ndarray):
    torch = torch_cuda()
    return dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


class DevicePool:
    """A canary-filled device pool laid out as the workload describes."""

    def __init__(self, W: wl.Workload, fmt: int | None = None, fill: int = CANARY):
        torch = torch_cuda()
        self.W = W
        self.fmt = W.kv_format if fmt is None else fmt
        self.page_bytes = wl.BYTES_PER_TOKEN[self.fmt] * W.page_size
        self.stride = max(W.page_stride_bytes, self.page_bytes)
        self.offset = W.offset_bytes
        self.num_pages = W.num_pages
        total = self.offset + self.num_pages * self.stride
        self.t = torch.full((total + 512,), fill, dtype=torch.uint8, device="cuda")
        shift = (-self.t.data_ptr()) % 256
        self.base = self.t[shift: shift + total]
        assert self.base.data_ptr() % 256 == 0
        self.pages2d = self.base[self.offset:].view(self.num_pages, self.stride)
        self.view = bd.make_pool(self.base, self.offset, self.stride, self.num_pages, W.page_size, self.fmt)

    def used_pids(self) -> np.ndarray:
        pt = self.W.page_table
        return np.unique(pt[pt >= 0]).astype(np.int64)

    def read_pages(self, pids: np.ndarray) -> np.ndarray:
        torch = torch_cuda()
        idx = torch.from_numpy(np.asarray(pids, np.int64)).to("cuda")
        return self.pages2d.index_select(0, idx).cpu().numpy()

    def write_pages(self, pids: np.ndarray, pages: np.ndarray) -> None:
        torch = torch_cuda()
        idx = torch.from_numpy(np.asarray(pids, np.int64)).to("cuda")
        src = torch.from_numpy(np.ascontiguousarray(pages)).to("cuda")
        self.pages2d[idx, : pages.shape[1]] = src


class CompactHostPool:
    """The oracle's copy of the used pages only, page c = the c-th used physical page
    in ascending order (page permutation is an invariant the oracle's tests pin)."""

    def __init__(self, W: wl.Workload, fmt: int | None = None, rows: np.ndarray | None = None):
        self.W = W
        self.fmt = W.kv_format if fmt is None else fmt
        P = W.page_size
        self.page_bytes = wl.BYTES_PER_TOKEN[self.fmt] * P
        pt = W.page_table
        self.pids = np.unique(pt[pt >= 0]).astype(np.int64)
        remap = np.full(W.num_pages, -1, np.int64)
        remap[self.pids] = np.arange(self.pids.size)
        self.page_table = np.where(pt >= 0, remap[np.maximum(pt, 0)], -1).astype(np.int32)
        self.pool = np.full(self.pids.size * self.page_bytes, CANARY, np.uint8)
        sel = np.arange(W.k_rows.shape[0]) if rows is None else rows
        slots = remap[W.slots[sel] // P] * P + W.slots[sel] % P
        oracle.k_store(self.pool, 0, self.page_bytes, self.pids.size, P, self.fmt, W.k_rows[sel], W.gamma, W.eps,
                       W.positions[sel], W.cos_sin, slots)

    def pages(self) -> np.ndarray:
        return self.pool.reshape(self.pids.size, self.page_bytes)


def oracle_q(W: wl.Workload, fmt: int):
    if fmt == wl.MXFP4:
        q, qs = oracle.q_quant_mxfp4(W.q_rows)
        return q, qs, W.w
    q8, w8 = oracle.q_quant_fp8(W.q_rows, W.w)
    return q8, None, w8


def oracle_logits(hp: CompactHostPool, q, qs, w, rows: np.ndarray | None, out_stride: int):
    W = hp.W
    return oracle.logits_paged(hp.pool, 0, hp.page_bytes, hp.pids.size, W.page_size, hp.fmt, q, qs, w,
                               hp.page_table, W.ctx, W.B, W.n_q, W.H, out_stride, rows)


def valid_mask(W: wl.Workload, rows: np.ndarray, stride: int) -> np.ndarray:
    n = np.array([W.valid_len(int(r)) for r in rows])
    return np.arange(stride)[None, :] < n[:, None]


def assert_logits_close(got: np.ndarray, ref: np.ndarray, mask: np.ndarray, label: str = "") -> dict:
    """The parity rule for logits: over the valid cells of the call,
    max|d| <= 1e-4 * max|ref| and cosine >= 0.999999."""
    g = got[mask].astype(np.float64)
    r = ref[mask]
    assert np.all(np.isfinite(g)), f"{label}: non-finite logits in valid cells"
    scale = np.abs(r).max()
    err = np.abs(g - r).max() if r.size else 0.0
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r))) if r.size and scale > 0 else 1.0
    assert err <= 1e-4 * scale, f"{label}: max|d| {err:.3e} > 1e-4 * {scale:.3e}"
    assert cos >= 0.999999, f"{label}: cosine {cos:.9f}"
    return {"max_abs_err": float(err), "max_abs_ref": float(scale), "rel": float(err / scale) if scale else 0.0,
            "cosine": cos}


def assert_topk_valid(got: np.ndarray, ref_logits: np.ndarray, W: wl.Workload, rows: np.ndarray, k: int,
                      tau: float, label: str = "") -> None:
    """The parity rule for top-k against fp64 logits: with v_k the oracle's k-th value,
    every token above v_k + tau is selected, none below v_k - tau, exactly min(k, n)
    distinct valid indices, and -1 only in the tail."""
    for i, r in enumerate(rows):
        n = W.valid_len(int(r))
        sel = got[i]
        m = min(k, n)
        assert np.all(sel[:m] >= 0) and np.all(sel[m:] == -1), f"{label} row {r}: padding"
        s = sel[:m]
        assert len(set(s.tolist())) == m and np.all(s < n), f"{label} row {r}: duplicates or masked"
        if n <= k:
            assert sorted(s.tolist()) == list(range(n)), f"{label} row {r}: short row"
            continue
        lv = ref_logits[i, :n]
        vk = np.sort(lv)[::-1][k - 1]
        must = np.where(lv > vk + tau)[0]
        never = np.where(lv < vk - tau)[0]
        ss = set(s.tolist())
        assert all(x in ss for x in must.tolist()), f"{label} row {r}: missing a clear winner"
        assert not any(x in ss for x in never.tolist()), f"{label} row {r}: selected a clear loser"
