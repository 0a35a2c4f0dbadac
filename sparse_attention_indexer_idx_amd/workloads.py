"""Seeded synthetic inputs for the lightning-indexer hot path.

This module draws inputs only: random bf16 rows, weights, context lengths, physical
page assignments, slot mappings and the rotary cos/sin table a model would hand the
K-cache store.  It holds none of the method's arithmetic (no norm, rotation,
quantisation, scoring or selection), so both the HIP path and the CPU oracle can take
their inputs from it.

The five workloads follow the shapes the pages report for the isolated scorer and the
DeepSeek-V4 / V4.1 indexer ("[ROCm][Perf] Add AITER paged MXFP4 sparse indexing on
gfx950", Performance and accuracy: decode B64/H32/D128/8K and prefill 8192 queries,
page size 128; "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose: 64 heads x 128,
top-k 1024, compress ratio 4, 64-entry pages, and Test Plan: max model length 9472 and
speculative decoding with several draft tokens).  Random values stand in for model
activations; nothing here comes from a dataset.

Recipe: numpy PCG64 seeded with 1000 + config index unless a seed is given; independent
child streams (SeedSequence.spawn) for K rows, Q rows, weights, lengths and pages.
bf16 values are fp32 N(0,1) draws rounded to nearest-even bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
ROPE_DIM = 64
GIB = 1 << 30

MXFP4 = 0
FP8 = 1
BYTES_PER_TOKEN = {MXFP4: 68, FP8: 132}  # "Dense MXFP4 indexer for DeepSeek-V4 on ROCm", Purpose


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rope_cos_sin(max_pos: int, base: float = 10000.0) -> np.ndarray:
    """The rotary table a NeoX-style rotary embedding caches: row p holds
    cos(p * theta_i) for i < 32, then sin(p * theta_i), theta_i = base^(-2i/64),
    computed in fp64 and stored as fp32 (shape [max_pos, 64])."""
    inv_freq = np.power(np.float64(base), -np.arange(0, ROPE_DIM, 2, dtype=np.float64) / ROPE_DIM)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclass
class Workload:
    """Everything one call of the hot path consumes (host arrays)."""
    name: str
    B: int
    n_q: int
    H: int
    page_size: int
    topk: int
    kv_format: int
    ctx: np.ndarray                 # int32 [B]
    num_pages: int
    offset_bytes: int
    page_stride_bytes: int
    page_table: np.ndarray          # int32 [B, max_pages_per_seq]; unused entries -1
    k_rows: np.ndarray              # uint16 bf16 bits [N, 128], sequences back to back
    k_seq: np.ndarray               # int32 [N] sequence of each K row
    positions: np.ndarray           # int32 [N] logical token index (= RoPE position)
    slots: np.ndarray               # int64 [N] page * page_size + row
    q_rows: np.ndarray              # uint16 bf16 bits [B, n_q, H, 128]
    w: np.ndarray                   # fp32 [B, n_q, H]
    gamma: np.ndarray               # fp32 [128]
    eps: float
    cos_sin: np.ndarray             # fp32 [max_pos, 64]
    seed: int
    notes: dict = field(default_factory=dict)

    @property
    def max_ctx(self) -> int:
        return int(self.ctx.max())

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def bytes_per_token(self) -> int:
        return BYTES_PER_TOKEN[self.kv_format]

    @property
    def page_bytes(self) -> int:
        return self.bytes_per_token * self.page_size

    @property
    def pool_bytes(self) -> int:
        return self.offset_bytes + self.num_pages * self.page_stride_bytes

    @property
    def rows(self) -> int:
        return self.B * self.n_q

    def valid_len(self, r: int) -> int:
        b, j = divmod(r, self.n_q)
        return int(min(max(int(self.ctx[b]) - self.n_q + 1 + j, 0), int(self.ctx[b])))

    def seq_row_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ctx.astype(np.int64))])


def _bf16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def _assign_pages(rng, ctx, page_size, num_pages, forced=()):
    """Distinct physical pages for every logical page, drawn from the whole pool,
    with the `forced` page ids included; returns the page table [B, max_pages]."""
    need = [(int(c) + page_size - 1) // page_size for c in ctx]
    total = int(sum(need))
    assert total <= num_pages
    if total == num_pages:
        pids = rng.permutation(num_pages)
    else:
        pids = rng.choice(num_pages, size=total, replace=False)
        forced = [f for f in forced if f not in set(pids.tolist())]
        for i, f in enumerate(forced):
            pids[i] = f
        pids = rng.permutation(pids)
    max_pages = max(need)
    pt = np.full((len(ctx), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        pt[b, :n] = pids[pos:pos + n]
        pos += n
    return pt


def _k_rows_for(ctx, page_table, page_size):
    seq = np.repeat(np.arange(len(ctx), dtype=np.int32), ctx)
    pos = np.concatenate([np.arange(int(c), dtype=np.int32) for c in ctx])
    pid = page_table[seq, pos // page_size].astype(np.int64)
    slots = pid * page_size + (pos % page_size)
    return seq, pos, slots


def straddling_pages(page_stride: int, offset: int = 0):
    """Page ids whose bytes span 2 GiB, 4 GiB, 4608 MiB and 4.608e9 B: the address
    boundaries at 2, 4 and 4.608 GB that the scorer's test coverage lists (page
    "[ROCm][Perf] Add AITER paged MXFP4 sparse indexing on gfx950", Test plan), with
    4.608 GB read both as binary and as decimal units."""
    out = []
    for boundary in (1 << 31, 1 << 32, 4608 << 20, 4_608_000_000):
        pid = (boundary - offset) // page_stride
        if (boundary - offset) % page_stride == 0:
            pid -= 1  # a page that starts exactly on the boundary does not straddle it
        out.append(int(pid))
    return out


CONFIG_NAMES = {
    0: "tiny decode B2/H4/ctx{200,256}/page64",
    1: "decode B64/H32/D128/ctx8192/page128",
    2: "prefill 8192 causal queries/H32/ctx8192/page128",
    3: "V4-Pro-style decode B128/n_q3/H64/ctx U[256,2368]/page64",
    4: "large-pool decode B256/H32/ctx U[4096,16384]/page128/6GiB pool",
}


def make_workload(config: int, kv_format: int = MXFP4, seed: int | None = None, *, gamma_random: bool = False,
                  scale: dict | None = None) -> Workload:
    """Build one of the five workloads.  `scale` may override B/ctx, and for the decode
    workloads the head count H and query tokens n_q, for test variants (e.g. {"B": 4});
    the default is the full shape."""
    seed = 1000 + config if seed is None else seed
    ss = np.random.SeedSequence(seed)
    r_k, r_q, r_w, r_len, r_pg, r_misc = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]
    scale = scale or {}
    bpt = BYTES_PER_TOKEN[kv_format]
    forced = ()
    if config == 0:
        B, n_q, H, P, k = 2, 1, 4, 64, 64
        ctx = np.array([200, 256], np.int32)
        num_pages, offset = 16, 0
        stride = bpt * P
        w_div = np.sqrt(H)
    elif config == 1:
        B, n_q, H, P, k = 64, 1, 32, 128, 1024
        ctx = np.full(B, 8192, np.int32)
        num_pages, offset, stride = 4096, 0, bpt * P
        w_div = np.sqrt(H)
    elif config == 2:
        B, n_q, H, P, k = 1, 8192, 32, 128, 1024
        ctx = np.array([8192], np.int32)
        num_pages, offset, stride = 64, 0, bpt * P
        w_div = np.sqrt(H)
    elif config == 3:
        B, n_q, H, P, k = 128, 3, 64, 64, 1024
        ctx = r_len.integers(256, 2368, size=B, endpoint=True).astype(np.int32)
        num_pages = int(sum((int(c) + P - 1) // P for c in ctx))
        stride = bpt * P + 256           # page stride larger than the page: a gap after each page
        offset = 3 * stride + 256        # nonzero start offset into the pool
        w_div = 8.0
    elif config == 4:
        B, n_q, H, P, k = 256, 1, 32, 128, 1024
        ctx = r_len.integers(4096, 16384, size=B, endpoint=True).astype(np.int32)
        stride, offset = bpt * P, 0
        num_pages = (6 * GIB - offset) // stride
        forced = straddling_pages(stride, offset)
        w_div = np.sqrt(H)
    else:
        raise ValueError(f"unknown config {config}")
    if "H" in scale:
        H = int(scale["H"])
        w_div = np.sqrt(H)
    if "n_q" in scale and config != 2:
        n_q = int(scale["n_q"])
    if "B" in scale:
        B = int(scale["B"])
        ctx = ctx[:B]
    if "ctx" in scale:
        ctx = np.minimum(ctx, int(scale["ctx"])).astype(np.int32)
        if config == 2:
            n_q = int(ctx[0])
    if config in (0, 1, 2):
        num_pages = max(num_pages, int(sum((int(c) + P - 1) // P for c in ctx)))
    pt = _assign_pages(r_pg, ctx, P, num_pages, forced)
    seq, pos, slots = _k_rows_for(ctx, pt, P)
    k_rows = _bf16_normal(r_k, (int(ctx.sum()), HEAD_DIM))
    q_rows = _bf16_normal(r_q, (B, n_q, H, HEAD_DIM))
    w = (r_w.standard_normal(size=(B, n_q, H)) / w_div).astype(np.float32)
    gamma = (np.ones(HEAD_DIM, np.float32) if not gamma_random
             else (1.0 + 0.25 * r_misc.standard_normal(HEAD_DIM)).astype(np.float32))
    return Workload(name=CONFIG_NAMES[config], B=B, n_q=n_q, H=H, page_size=P, topk=k, kv_format=kv_format, ctx=ctx,
                    num_pages=int(num_pages), offset_bytes=int(offset), page_stride_bytes=int(stride), page_table=pt,
                    k_rows=k_rows, k_seq=seq, positions=pos, slots=slots, q_rows=q_rows, w=w, gamma=gamma,
                    eps=1e-6, cos_sin=rope_cos_sin(int(ctx.max())), seed=seed,
                    notes={"config": config, "forced_pages": list(forced)})


def random_logits(rng: np.random.Generator, rows: int, stride: int, *, ties: bool = False) -> np.ndarray:
    """fp32 logits rows for the top-k unit tests; with `ties`, values are drawn from a
    small set so that equal values are common (and include both signed zeros)."""
    if not ties:
        return rng.standard_normal(size=(rows, stride), dtype=np.float32)
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0], np.float32)
    return vals[rng.integers(0, vals.size, size=(rows, stride))]


def candidate_blocks(rng: np.random.Generator, W: Workload, n_cand: int, *, pad: int = 0,
                     past_table: int = 0, shuffled: bool = False) -> np.ndarray:
    """Candidate block ids [rows, n_cand] int32 for the candidate-block scorer: per row,
    distinct block (page-table) indices of its sequence drawn without replacement from
    the blocks that hold tokens (ascending unless `shuffled`); when a sequence has fewer
    blocks, the rest are padding (-1).  `pad` entries per row are then replaced by -1 and
    `past_table` by ids at or past the page-table width (edge cases)."""
    P, mp = W.page_size, W.page_table.shape[1]
    out = np.full((W.rows, n_cand), -1, np.int32)
    for r in range(W.rows):
        nb = min(mp, -(-int(W.ctx[r // W.n_q]) // P))
        m = min(n_cand, nb)
        ids = rng.choice(nb, m, replace=False) if m else np.zeros(0, np.int64)
        out[r, :m] = np.sort(ids) if not shuffled else ids
        if pad:
            out[r, rng.choice(n_cand, pad, replace=False)] = -1
        if past_table:
            out[r, rng.choice(n_cand, past_table, replace=False)] = mp + rng.integers(0, 3, past_table)
    return out
