"""ctypes binding of libidx.so (include/idx.h) — argument marshalling only.

Each function carries the name of the C entry point it calls and takes torch tensors
that already live on the current HIP device; it passes their data pointers, sizes and
the current stream to the library and raises IdxError on a nonzero status.  No step of
the hot path runs here: the work is done by the HIP kernels in the library.  If the
library is missing the first call raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libidx.so")

IDX_OK, IDX_EINVAL, IDX_EUNSUPPORTED, IDX_EALIGN, IDX_EHIP, IDX_ESCRATCH = 0, -1, -2, -3, -4, -5
IDX_NOALLOC_MAX_SEQS = 16384
IDX_KV_MXFP4, IDX_KV_FP8_E4M3 = 0, 1

EXPORTS = ("idx_k_store_mxfp4", "idx_k_store_fp8", "idx_qk_prep_fp8", "idx_q_prep_mxfp4", "idx_q_quant_mxfp4", "idx_q_quant_fp8",
           "idx_logits_paged", "idx_logits_candidates", "idx_topk_candidates",
           "idx_topk", "idx_workspace_bytes", "idx_decode_step", "idx_decode_step_noalloc", "idx_decode_step_fused", "idx_diag_fp64", "idx_diag_mfma", "idx_diag_hbm_read",
           "idx_device_info", "idx_bytes_per_token", "idx_device_check", "idx_status_string")


class IdxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class IdxPool(ctypes.Structure):
    """Mirror of idx_pool."""
    _fields_ = [("base", ctypes.c_void_p), ("offset_bytes", ctypes.c_int64), ("page_stride_bytes", ctypes.c_int64),
                ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32), ("kv_format", ctypes.c_int32)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libidx.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} not found: build it with `python -m sparse_attention_indexer_idx_amd.build`")
    # torch first: the library then binds to the HIP runtime torch already loaded, so the
    # two share one runtime (devices, streams and allocations), whatever the import order.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    V, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    PP = ctypes.POINTER(IdxPool)
    sigs = {
        "idx_k_store_mxfp4": [PP, V, I64, I64, V, F32, V, V, I32, V, V],
        "idx_k_store_fp8": [PP, V, I64, I64, V, F32, V, V, I32, V, V],
        "idx_q_quant_mxfp4": [V, I64, V, V, V],
        "idx_q_prep_mxfp4": [V, I64, I32, V, V, I32, V, F32, V, V, V, V],
        "idx_qk_prep_fp8": [PP, V, V, I64, I32, V, V, V, I32, I32, V, V, F32, V, V, V, V],
        "idx_q_quant_fp8": [V, V, I64, V, V, V],
        "idx_logits_paged": [PP, V, V, V, V, I32, V, I32, I32, I32, I32, I32, V, I64, V, ctypes.c_size_t, V],
        "idx_topk": [V, I64, V, I32, I32, I32, V, V, ctypes.c_size_t, V],
        "idx_workspace_bytes": [I32, I32, I32, I32, I32],
        "idx_logits_candidates": [PP, V, V, V, V, I32, V, I32, I32, I32, I32, V, I32, V, I64, V],
        "idx_topk_candidates": [V, I64, V, I32, I32, I32, I32, I32, V, V],
        "idx_decode_step_fused": [I32, I32, I32, I32],
        "idx_decode_step_noalloc": [PP, V, I64, V, F32, V, V, I32, V, V, V, V, V, I32, V, I32, I32, I32, I32, I32, V,
                                    I64, I32, V, V],
        "idx_decode_step": [PP, V, I64, V, F32, V, V, I32, V, V, V, V, V, I32, V, I32, I32, I32, I32, I32, V, I64, I32,
                            V, V, ctypes.c_size_t, V],
        "idx_diag_fp64": [V, V, V, V, I64, V],
        "idx_diag_mfma": [I32, I32, I32, V, V],
        "idx_diag_hbm_read": [V, I64, I32, V, V],
        "idx_device_info": [V, V],
        "idx_bytes_per_token": [I32],
        "idx_device_check": [],
        "idx_status_string": [ctypes.c_int],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.idx_bytes_per_token.restype = ctypes.c_int64
    lib.idx_workspace_bytes.restype = ctypes.c_size_t
    lib.idx_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().idx_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != IDX_OK:
        raise IdxError(fn, status, status_string(status))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_pool(base, offset_bytes: int, page_stride_bytes: int, num_pages: int, page_size: int,
              kv_format: int) -> IdxPool:
    """An idx_pool view over the uint8 device tensor `base` (the caller keeps it alive)."""
    return IdxPool(base.data_ptr(), offset_bytes, page_stride_bytes, num_pages, page_size, kv_format)


def idx_k_store_mxfp4(pool: IdxPool, k_bf16, gamma, eps: float, positions, cos_sin, slot_mapping, stream=None):
    _check("idx_k_store_mxfp4", load().idx_k_store_mxfp4(
        ctypes.byref(pool), _ptr(k_bf16), k_bf16.shape[0], k_bf16.stride(0), _ptr(gamma), eps, _ptr(positions),
        _ptr(cos_sin), cos_sin.shape[0], _ptr(slot_mapping), _stream(stream)))


def idx_k_store_fp8(pool: IdxPool, k_bf16, gamma, eps: float, positions, cos_sin, slot_mapping, stream=None):
    _check("idx_k_store_fp8", load().idx_k_store_fp8(
        ctypes.byref(pool), _ptr(k_bf16), k_bf16.shape[0], k_bf16.stride(0), _ptr(gamma), eps, _ptr(positions),
        _ptr(cos_sin), cos_sin.shape[0], _ptr(slot_mapping), _stream(stream)))


def idx_q_prep_mxfp4(q_bf16, positions, cos_sin, w, w_scale: float, q_packed, q_scale, w_out, stream=None):
    """q_bf16 [T, H, 128] bf16, positions [T] int32, w [T, H] fp32."""
    T, H = q_bf16.shape[0], q_bf16.shape[1]
    _check("idx_q_prep_mxfp4", load().idx_q_prep_mxfp4(
        _ptr(q_bf16), T, H, _ptr(positions), _ptr(cos_sin), cos_sin.shape[0], _ptr(w), w_scale, _ptr(q_packed),
        _ptr(q_scale), _ptr(w_out), _stream(stream)))


def idx_q_quant_mxfp4(q_bf16, q_packed, q_scale, stream=None):
    n = q_bf16.numel() // 128
    _check("idx_q_quant_mxfp4", load().idx_q_quant_mxfp4(_ptr(q_bf16), n, _ptr(q_packed), _ptr(q_scale),
                                                         _stream(stream)))


def idx_qk_prep_fp8(pool: IdxPool, q_bf16, k_bf16, w, positions, cos_sin, neox: bool, ln_gamma, ln_beta,
                    eps: float, slot_mapping, q_fp8, w_out, stream=None):
    """q_bf16 [T, H, 128] and k_bf16 [T, 128] bf16, w [T, H] fp32 -> q_fp8 [T, H, 128] uint8,
    w_out [T, H] fp32, and the K rows stored into the FP8 pool."""
    T, H = q_bf16.shape[0], q_bf16.shape[1]
    _check("idx_qk_prep_fp8", load().idx_qk_prep_fp8(
        ctypes.byref(pool), _ptr(q_bf16), _ptr(k_bf16), T, H, _ptr(w), _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], 1 if neox else 0, _ptr(ln_gamma), _ptr(ln_beta), eps, _ptr(slot_mapping), _ptr(q_fp8),
        _ptr(w_out), _stream(stream)))


def idx_q_quant_fp8(q_bf16, w, q_fp8, w_out, stream=None):
    n = q_bf16.numel() // 128
    _check("idx_q_quant_fp8", load().idx_q_quant_fp8(_ptr(q_bf16), _ptr(w), n, _ptr(q_fp8), _ptr(w_out),
                                                     _stream(stream)))


def _ws(workspace) -> tuple[int | None, int]:
    return (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())


def idx_workspace_bytes(B: int, n_q: int, H: int, max_ctx: int, k: int) -> int:
    return int(load().idx_workspace_bytes(B, n_q, H, max_ctx, k))


def idx_logits_paged(pool: IdxPool, q, q_scale, w, page_table, ctx_lens, B: int, n_q: int, H: int, max_ctx: int,
                     logits, workspace=None, stream=None):
    ws, wsb = _ws(workspace)
    _check("idx_logits_paged", load().idx_logits_paged(
        ctypes.byref(pool), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(page_table), page_table.shape[1], _ptr(ctx_lens),
        B, n_q, H, 128, max_ctx, _ptr(logits), logits.stride(0), ws, wsb, _stream(stream)))


def idx_logits_candidates(pool: IdxPool, q, q_scale, w, page_table, ctx_lens, B: int, n_q: int, H: int, cand_blocks,
                          logits, stream=None):
    """cand_blocks: int32 [B*n_q][n_cand] block (page-table) indices, negative = padding;
    logits: fp32 [B*n_q][>= n_cand*P]."""
    _check("idx_logits_candidates", load().idx_logits_candidates(
        ctypes.byref(pool), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(page_table), page_table.shape[1], _ptr(ctx_lens),
        B, n_q, H, 128, _ptr(cand_blocks), cand_blocks.shape[1], _ptr(logits), logits.stride(0), _stream(stream)))


def idx_topk_candidates(logits, cand_blocks, page_size: int, B: int, n_q: int, k: int, out_idx, stream=None):
    _check("idx_topk_candidates", load().idx_topk_candidates(
        _ptr(logits), logits.stride(0), _ptr(cand_blocks), cand_blocks.shape[1], page_size, B, n_q, k, _ptr(out_idx),
        _stream(stream)))


def idx_topk(logits, ctx_lens, B: int, n_q: int, k: int, out_idx, workspace=None, stream=None):
    """logits [B*n_q][stride] fp32 (the stride bounds the row length), out_idx [B*n_q][k] int32."""
    ws, wsb = _ws(workspace)
    _check("idx_topk", load().idx_topk(_ptr(logits), logits.stride(0), _ptr(ctx_lens), B, n_q, k, _ptr(out_idx), ws,
                                       wsb, _stream(stream)))


def idx_decode_step_fused(B: int, n_q: int, H: int, max_ctx: int) -> int:
    """1 if idx_decode_step runs this shape as the one fused kernel, 0 if as three kernels."""
    r = int(load().idx_decode_step_fused(B, n_q, H, max_ctx))
    if r < 0:
        _check("idx_decode_step_fused", r)
    return r


def idx_decode_step(pool: IdxPool, k_bf16, gamma, eps: float, positions, cos_sin, slot_mapping, q, q_scale, w,
                    page_table, ctx_lens, B: int, n_q: int, H: int, max_ctx: int, logits, k: int, out_idx, workspace,
                    stream=None):
    """k_bf16 / positions / slot_mapping hold the B*n_q new rows (row b*n_q + j is token
    ctx[b] - n_q + j of sequence b); workspace is a zero-filled device buffer of at least
    idx_workspace_bytes(B, n_q, H, max_ctx, k) bytes."""
    _check("idx_decode_step", load().idx_decode_step(
        ctypes.byref(pool), _ptr(k_bf16), k_bf16.stride(0), _ptr(gamma), eps, _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(page_table), page_table.shape[1],
        _ptr(ctx_lens), B, n_q, H, 128, max_ctx, _ptr(logits), logits.stride(0), k, _ptr(out_idx), *_ws(workspace),
        _stream(stream)))


def idx_decode_step_noalloc(pool: IdxPool, k_bf16, gamma, eps: float, positions, cos_sin, slot_mapping, q, q_scale,
                            w, page_table, ctx_lens, B: int, n_q: int, H: int, max_ctx: int, logits, k: int, out_idx,
                            stream=None):
    """idx_decode_step without a workspace: the block counters live in the library's own
    static device array (B <= IDX_NOALLOC_MAX_SEQS)."""
    _check("idx_decode_step_noalloc", load().idx_decode_step_noalloc(
        ctypes.byref(pool), _ptr(k_bf16), k_bf16.stride(0), _ptr(gamma), eps, _ptr(positions), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), _ptr(q), _ptr(q_scale), _ptr(w), _ptr(page_table), page_table.shape[1],
        _ptr(ctx_lens), B, n_q, H, 128, max_ctx, _ptr(logits), logits.stride(0), k, _ptr(out_idx), _stream(stream)))


def idx_diag_fp64(a, b, quot, root, stream=None):
    _check("idx_diag_fp64", load().idx_diag_fp64(_ptr(a), _ptr(b), _ptr(quot), _ptr(root), a.numel(),
                                                 _stream(stream)))


def idx_diag_mfma(fmt: int, blocks: int, rounds: int, out, stream=None):
    _check("idx_diag_mfma", load().idx_diag_mfma(fmt, blocks, rounds, _ptr(out), _stream(stream)))


def idx_diag_hbm_read(buf, blocks: int, out, stream=None):
    """Plain streaming read of the whole of `buf` (bytes a multiple of 16)."""
    _check("idx_diag_hbm_read", load().idx_diag_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), blocks,
                                                         _ptr(out), _stream(stream)))


def idx_device_info() -> tuple[int, int]:
    """(compute units, peak shader clock in kHz) of the current device."""
    cus, khz = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("idx_device_info", load().idx_device_info(ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value


def idx_bytes_per_token(kv_format: int) -> int:
    return int(load().idx_bytes_per_token(kv_format))


def idx_device_check() -> int:
    return int(load().idx_device_check())
