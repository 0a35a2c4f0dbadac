"""Oracle for the lightning-indexer hot path — TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU implementation (``idx_oracle.c``) of what the hot path computes:
the MXFP4 / FP8 codecs, the K-cache store (RMSNorm -> NeoX RoPE -> quantise -> page
store), the Q packing and the MXFP4 Q preparation (NeoX RoPE -> pack -> weight fold),
the FP8 QK preparation (LayerNorm on k, NeoX or interleaved RoPE on q and k, FP8 k to
the pages, per-vector FP8 q with its scale folded into the weights, padding rows
zeroed), the paged MQA logits with the causal/length mask, the per-row top-k, and both
restricted to a row's candidate blocks.
Each C function cites the page passage it follows.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and never imports it.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, exhaustive or brute-force checks and invariants.  Parity unpinned: the
absolute logits at realistic shapes rest only on those checks (the pages print no
numeric example); the FP8 scale rule (amax / 448) is a reading, not a printed value.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "idx_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_MXFP4 = 0
FMT_FP8 = 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no contraction, no fast-math, OpenMP)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P, I64, I32, F32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
            sig = {
                "orc_e2m1_decode": (D, [ctypes.c_uint]),
                "orc_e8m0_decode": (D, [ctypes.c_uint]),
                "orc_e4m3_decode": (D, [ctypes.c_uint]),
                "orc_e4m3_encode": (ctypes.c_uint8, [D]),
                "orc_mxfp4_quant_block": (None, [P, P, P]),
                "orc_bytes_per_token": (I64, [ctypes.c_int]),
                "orc_num_threads": (ctypes.c_int, []),
                "orc_k_store": (ctypes.c_int, [P, I64, I64, I64, I32, I32, P, I64, I64, P, F32, P, P, I32, P]),
                "orc_k_rows_exact": (None, [P, I64, I64, P, F32, P, P, P]),
                "orc_q_quant_mxfp4": (None, [P, I64, P, P]),
                "orc_q_quant_fp8": (None, [P, P, I64, P, P]),
                "orc_q_prep_mxfp4": (None, [P, I64, I32, P, P, I32, P, F32, P, P, P]),
                "orc_qk_prep_fp8": (ctypes.c_int, [P, I64, I64, I64, I32, P, P, I64, I32, P, P, P, I32, I32, P, P,
                                                   F32, P, P, P]),
                "orc_valid_len": (I64, [P, I32, I64]),
                "orc_logits_paged": (ctypes.c_int, [P, I64, I64, I64, I32, I32, P, P, P, P, I32, P, I32, I32, I32,
                                                    P, I64, P, I64]),
                "orc_logits_exact": (None, [P, P, P, I64, P, I32, I32, I32, P, I64, P, I64]),
                "orc_topk": (None, [P, I64, P, I32, I32, P, I64, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- codecs
def e2m1_decode(nibble: int) -> float:
    return _load().orc_e2m1_decode(int(nibble))


def e8m0_decode(byte: int) -> float:
    return _load().orc_e8m0_decode(int(byte))


def e4m3_decode(byte: int) -> float:
    return _load().orc_e4m3_decode(int(byte))


def e4m3_encode(v: float) -> int:
    return int(_load().orc_e4m3_encode(float(v)))


def mxfp4_quant_block(v) -> tuple[bytes, int]:
    """Quantise 32 fp64 values: (16 packed nibble bytes, E8M0 scale byte)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.shape == (32,)
    nib = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    _load().orc_mxfp4_quant_block(_p(v), _p(nib), _p(sc))
    return nib.tobytes(), int(sc[0])


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_num_threads())


def bytes_per_token(fmt: int) -> int:
    return int(_load().orc_bytes_per_token(fmt))


# ----------------------------------------------------------------------------- K store
def k_store(pool: np.ndarray, offset: int, stride: int, num_pages: int, page_size: int, fmt: int,
            k_bf16: np.ndarray, gamma: np.ndarray, eps: float, positions: np.ndarray, cos_sin: np.ndarray,
            slots: np.ndarray) -> None:
    """Write K rows into a host pool (uint8 array) in place."""
    assert pool.dtype == np.uint8 and k_bf16.dtype == np.uint16 and k_bf16.shape[1] == 128
    k_bf16 = np.ascontiguousarray(k_bf16)
    gamma = np.ascontiguousarray(gamma, np.float32)
    positions = np.ascontiguousarray(positions, np.int32)
    cos_sin = np.ascontiguousarray(cos_sin, np.float32)
    slots = np.ascontiguousarray(slots, np.int64)
    rc = _load().orc_k_store(_p(pool), offset, stride, num_pages, page_size, fmt, _p(k_bf16), k_bf16.shape[0], 128,
                             _p(gamma), float(eps), _p(positions), _p(cos_sin), cos_sin.shape[0], _p(slots))
    if rc != 0:
        raise ValueError("oracle k_store: invalid slot or position")


def k_rows_exact(k_bf16, gamma, eps, positions, cos_sin) -> np.ndarray:
    k_bf16 = np.ascontiguousarray(k_bf16, np.uint16)
    out = np.empty((k_bf16.shape[0], 128), np.float64)
    _load().orc_k_rows_exact(_p(k_bf16), k_bf16.shape[0], 128, _p(np.ascontiguousarray(gamma, np.float32)),
                             float(eps), _p(np.ascontiguousarray(positions, np.int32)),
                             _p(np.ascontiguousarray(cos_sin, np.float32)), _p(out))
    return out


# ----------------------------------------------------------------------------- Q quant
def q_quant_mxfp4(q_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """q_bf16 [..., 128] uint16 -> (packed [..., 64] uint8, scales [..., 4] uint8)."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    n = q.size // 128
    qp = np.empty(q.shape[:-1] + (64,), np.uint8)
    qs = np.empty(q.shape[:-1] + (4,), np.uint8)
    _load().orc_q_quant_mxfp4(_p(q), n, _p(qp), _p(qs))
    return qp, qs


def q_prep_mxfp4(q_bf16: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, w: np.ndarray,
                 w_scale: float) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q_bf16 [T, H, 128] uint16, positions [T], w [T, H] -> (packed [T, H, 64] uint8,
    scales [T, H, 4] uint8, w_out [T, H] fp32): rotation, MXFP4 packing, weight fold."""
    q_bf16 = np.ascontiguousarray(q_bf16, np.uint16)
    T, H = q_bf16.shape[0], q_bf16.shape[1]
    assert q_bf16.shape[2] == 128
    cos_sin = np.ascontiguousarray(cos_sin, np.float32)
    out = np.empty((T, H, 64), np.uint8)
    sc = np.empty((T, H, 4), np.uint8)
    wo = np.empty((T, H), np.float32)
    _load().orc_q_prep_mxfp4(_p(q_bf16), T, H, _p(np.ascontiguousarray(positions, np.int32)), _p(cos_sin),
                             cos_sin.shape[0], _p(np.ascontiguousarray(w, np.float32)), w_scale, _p(out), _p(sc),
                             _p(wo))
    return out, sc, wo


def q_quant_fp8(q_bf16: np.ndarray, w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """q_bf16 [..., H, 128], w [..., H] -> (e4m3 codes [..., H, 128], w with q scale folded)."""
    q = np.ascontiguousarray(q_bf16, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    n = q.size // 128
    assert w.size == n
    q8 = np.empty(q.shape, np.uint8)
    wo = np.empty(w.shape, np.float32)
    _load().orc_q_quant_fp8(_p(q), _p(w), n, _p(q8), _p(wo))
    return q8, wo


def qk_prep_fp8(pool: np.ndarray, offset: int, stride: int, num_pages: int, page_size: int, q_bf16: np.ndarray,
                k_bf16: np.ndarray, w: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, neox: bool,
                ln_gamma: np.ndarray, ln_beta: np.ndarray, eps: float,
                slots: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """FP8 QK preparation: q_bf16 [T, H, 128], k_bf16 [T, 128] uint16, w [T, H] fp32.
    Writes the K rows into the host FP8 pool in place; returns (q codes [T, H, 128] uint8,
    w_out [T, H] fp32)."""
    q_bf16 = np.ascontiguousarray(q_bf16, np.uint16)
    k_bf16 = np.ascontiguousarray(k_bf16, np.uint16)
    T, H = q_bf16.shape[0], q_bf16.shape[1]
    assert q_bf16.shape[2] == 128 and k_bf16.shape == (T, 128) and pool.dtype == np.uint8
    cos_sin = np.ascontiguousarray(cos_sin, np.float32)
    q8 = np.empty((T, H, 128), np.uint8)
    wo = np.empty((T, H), np.float32)
    rc = _load().orc_qk_prep_fp8(_p(pool), offset, stride, num_pages, page_size, _p(q_bf16), _p(k_bf16), T, H,
                                 _p(np.ascontiguousarray(w, np.float32)),
                                 _p(np.ascontiguousarray(positions, np.int32)), _p(cos_sin), cos_sin.shape[0],
                                 1 if neox else 0, _p(np.ascontiguousarray(ln_gamma, np.float32)),
                                 _p(np.ascontiguousarray(ln_beta, np.float32)), float(eps),
                                 _p(np.ascontiguousarray(slots, np.int64)), _p(q8), _p(wo))
    if rc != 0:
        raise ValueError("oracle qk_prep_fp8: invalid arguments")
    return q8, wo


# ----------------------------------------------------------------------------- scorer
def valid_len(ctx: np.ndarray, n_q: int, r: int) -> int:
    ctx = np.ascontiguousarray(ctx, np.int32)
    return int(_load().orc_valid_len(_p(ctx), n_q, r))


def logits_paged(pool: np.ndarray, offset: int, stride: int, num_pages: int, page_size: int, fmt: int,
                 q: np.ndarray, q_scale: np.ndarray | None, w: np.ndarray, page_table: np.ndarray,
                 ctx: np.ndarray, B: int, n_q: int, H: int, out_stride: int,
                 rows: np.ndarray | None = None) -> np.ndarray:
    """fp64 logits [len(rows), out_stride]; cells s >= n_r are NaN."""
    q = np.ascontiguousarray(q, np.uint8)
    w = np.ascontiguousarray(w, np.float32)
    pt = np.ascontiguousarray(page_table, np.int32)
    ctx = np.ascontiguousarray(ctx, np.int32)
    if rows is None:
        rows = np.arange(B * n_q, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, out_stride), np.float64)
    qs = None if q_scale is None else np.ascontiguousarray(q_scale, np.uint8)
    rc = _load().orc_logits_paged(_p(pool), offset, stride, num_pages, page_size, fmt, _p(q), _p(qs), _p(w), _p(pt),
                                  pt.shape[1], _p(ctx), B, n_q, H, _p(rows), rows.size, _p(out), out_stride)
    if rc != 0:
        raise ValueError("oracle logits: page id outside the pool")
    return out


def logits_exact(q_rows: np.ndarray, w: np.ndarray, k_rows: np.ndarray, ctx: np.ndarray, n_q: int, H: int,
                 out_stride: int, rows: np.ndarray) -> np.ndarray:
    """Unquantised fp64 logits; q_rows [R, H, 128] fp64, k_rows [B, S, 128] fp64."""
    q_rows = np.ascontiguousarray(q_rows, np.float64)
    k_rows = np.ascontiguousarray(k_rows, np.float64)
    w = np.ascontiguousarray(w, np.float32)
    ctx = np.ascontiguousarray(ctx, np.int32)
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, out_stride), np.float64)
    _load().orc_logits_exact(_p(q_rows), _p(w), _p(k_rows), k_rows.shape[1] * 128, _p(ctx), k_rows.shape[0], n_q, H,
                             _p(rows), rows.size, _p(out), out_stride)
    return out


# ----------------------------------------------------------------------------- top-k
def candidate_cells(cand_blocks: np.ndarray, page_size: int, max_pages: int, ctx: np.ndarray, n_q: int):
    """Token index and validity of every candidate cell: row r, candidate j, cell i is
    token cand_blocks[r, j] * P + i, valid when the block id lies in [0, max_pages) and
    the token is below the row's valid length.  Returns (tokens [rows, n_cand*P] int64,
    valid bool of the same shape).  Reading of the two-level indexer's second level
    ([p2] Purpose: the candidate-pool path scores only the candidate blocks of a row):
    a candidate block is a page-sized run of the sequence's tokens, named by its index in
    the sequence's page table."""
    cand = np.asarray(cand_blocks, np.int64)
    rows, n_cand = cand.shape
    i = np.arange(page_size, dtype=np.int64)
    tok = (cand[:, :, None] * page_size + i[None, None, :]).reshape(rows, n_cand * page_size)
    n = np.array([valid_len(ctx, n_q, r) for r in range(rows)], np.int64)
    ok = ((cand >= 0) & (cand < max_pages))[:, :, None].repeat(page_size, axis=2).reshape(rows, -1)
    return tok, ok & (tok < n[:, None]) & (tok >= 0)


def logits_candidates(dense_logits: np.ndarray, cand_blocks: np.ndarray, page_size: int, max_pages: int,
                      ctx: np.ndarray, n_q: int) -> np.ndarray:
    """The scorer restricted to candidate cells: cell (r, j*P + i) holds the plain logit of
    its token (dense_logits from logits_paged for every row), -inf where the cell is not
    a valid candidate."""
    tok, ok = candidate_cells(cand_blocks, page_size, max_pages, ctx, n_q)
    out = np.full(tok.shape, -np.inf)
    r = np.nonzero(ok)
    out[r] = dense_logits[r[0], tok[r]]
    return out


def topk_candidates(cand_logits: np.ndarray, cand_blocks: np.ndarray, page_size: int, max_pages: int,
                    ctx: np.ndarray, n_q: int, k: int) -> np.ndarray:
    """Per row, the k tokens with the largest logits among the valid candidate cells
    (ties to the smaller token index), then -1."""
    tok, ok = candidate_cells(cand_blocks, page_size, max_pages, ctx, n_q)
    out = np.full((tok.shape[0], k), -1, np.int32)
    for r in range(tok.shape[0]):
        v, t = cand_logits[r][ok[r]], tok[r][ok[r]]
        order = np.lexsort((t, -v))[:k]
        out[r, :order.size] = t[order]
    return out


def topk(logits: np.ndarray, ctx: np.ndarray, n_q: int, k: int, rows: np.ndarray | None = None) -> np.ndarray:
    """Indices [len(rows), k] in rank order (logit desc, index asc), -1 padded.

    ``logits`` row i belongs to logical row rows[i] (fp32 inputs are widened exactly)."""
    lg = np.ascontiguousarray(logits, np.float64)
    ctx = np.ascontiguousarray(ctx, np.int32)
    if rows is None:
        rows = np.arange(lg.shape[0], dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, k), np.int32)
    _load().orc_topk(_p(lg), lg.shape[1], _p(ctx), n_q, k, _p(rows), rows.size, _p(out))
    return out
