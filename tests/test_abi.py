"""The C ABI without a GPU: the library loads, exports every function include/idx.h
declares, and rejects bad arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

from sparse_attention_indexer_idx_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")

FAKE = 0x7F0000000000  # 256-aligned; never dereferenced (validation fails first, or no device)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*|size_t)\s+(idx_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from sparse_attention_indexer_idx_amd import build
        build.build(verbose=False)
    return bd.load()


def no_gpu(lib):
    return lib.idx_device_check() != bd.IDX_OK


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("idx_k_store_mxfp4", "idx_logits_paged", "idx_topk", "idx_status_string"):
        assert n in names
    assert set(names) == set(bd.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(bd.status_string(st), str) and bd.status_string(st)


def test_bytes_per_token(lib):
    assert bd.idx_bytes_per_token(0) == 68 and bd.idx_bytes_per_token(1) == 132 and bd.idx_bytes_per_token(5) == -1


def pool(**kw):
    d = dict(base=FAKE, offset_bytes=0, page_stride_bytes=68 * 64, num_pages=16, page_size=64, kv_format=0)
    d.update(kw)
    return bd.IdxPool(d["base"], d["offset_bytes"], d["page_stride_bytes"], d["num_pages"], d["page_size"],
                      d["kv_format"])


def logits_call(lib, p=None, **kw):
    a = dict(q=FAKE, qs=FAKE, w=FAKE, pt=FAKE, maxp=4, ctx=FAKE, B=2, n_q=1, H=4, D=128, max_ctx=256,
             logits=FAKE, lstride=256)
    a.update(kw)
    p = p or pool()
    return lib.idx_logits_paged(ctypes.byref(p), a["q"], a["qs"], a["w"], a["pt"], a["maxp"], a["ctx"], a["B"],
                                a["n_q"], a["H"], a["D"], a["max_ctx"], a["logits"], a["lstride"], a.get("ws"),
                                ctypes.c_size_t(a.get("wsb", 0)), None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=64), bd.IDX_EUNSUPPORTED),
    (dict(H=0), bd.IDX_EINVAL),
    (dict(H=129), bd.IDX_EUNSUPPORTED),
    (dict(B=0), bd.IDX_EINVAL),
    (dict(n_q=0), bd.IDX_EINVAL),
    (dict(q=None), bd.IDX_EINVAL),
    (dict(qs=None), bd.IDX_EINVAL),          # MXFP4 needs scales
    (dict(max_ctx=257), bd.IDX_EINVAL),      # > max_pages * P and > stride
    (dict(lstride=100), bd.IDX_EINVAL),      # < max_ctx
    (dict(max_ctx=-1), bd.IDX_EINVAL),
    (dict(q=FAKE + 8), bd.IDX_EALIGN),
    (dict(ws=None, wsb=256), bd.IDX_EINVAL),         # a size with no buffer
    (dict(ws=FAKE + 64, wsb=256), bd.IDX_EALIGN),    # scratch must be 256-byte aligned
])
def test_logits_argument_checks(lib, kw, want):
    assert logits_call(lib, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(page_size=48 + 1), bd.IDX_EUNSUPPORTED),
    (dict(page_size=48), bd.IDX_EUNSUPPORTED),                   # a multiple of 16, not a power of two
    (dict(page_size=8), bd.IDX_EUNSUPPORTED),
    (dict(page_size=2048, page_stride_bytes=68 * 2048), bd.IDX_EUNSUPPORTED),
    (dict(page_stride_bytes=68 * 64 - 256), bd.IDX_EINVAL),     # smaller than a page
    (dict(page_stride_bytes=68 * 64 + 16), bd.IDX_EALIGN),
    (dict(offset_bytes=128), bd.IDX_EALIGN),
    (dict(offset_bytes=-256), bd.IDX_EINVAL),
    (dict(num_pages=0), bd.IDX_EINVAL),
    (dict(kv_format=3), bd.IDX_EINVAL),
    (dict(base=0), bd.IDX_EINVAL),
    (dict(base=FAKE + 64), bd.IDX_EALIGN),
    (dict(kv_format=1), bd.IDX_EINVAL),                          # FP8 page needs 132 B/token
    (dict(num_pages=1 << 62, page_stride_bytes=1 << 20), bd.IDX_EINVAL),
])
def test_pool_checks(lib, kw, want):
    assert logits_call(lib, p=pool(**kw)) == want


def test_k_store_checks(lib):
    P = pool()
    args = lambda **kw: dict(dict(k=FAKE, n=10, rs=128, g=FAKE, eps=1e-6, pos=FAKE, cs=FAKE, mp=512, sl=FAKE), **kw)
    def call(fn, p=P, **kw):
        a = args(**kw)
        return fn(ctypes.byref(p), a["k"], a["n"], a["rs"], a["g"], a["eps"], a["pos"], a["cs"], a["mp"], a["sl"], None)
    assert call(lib.idx_k_store_mxfp4, rs=64) == bd.IDX_EINVAL
    assert call(lib.idx_k_store_mxfp4, n=-1) == bd.IDX_EINVAL
    assert call(lib.idx_k_store_mxfp4, eps=0.0) == bd.IDX_EINVAL
    assert call(lib.idx_k_store_mxfp4, mp=0) == bd.IDX_EINVAL
    assert call(lib.idx_k_store_mxfp4, sl=None) == bd.IDX_EINVAL
    assert call(lib.idx_k_store_fp8) == bd.IDX_EINVAL            # an MXFP4 pool handed to the FP8 store
    assert call(lib.idx_k_store_mxfp4, p=pool(kv_format=1, page_stride_bytes=132 * 64)) == bd.IDX_EINVAL


def topk_call(lib, **kw):
    a = dict(lg=FAKE, ls=256, ctx=FAKE, B=2, n_q=1, k=64, out=FAKE, ws=None, wsb=0)
    a.update(kw)
    return lib.idx_topk(a["lg"], a["ls"], a["ctx"], a["B"], a["n_q"], a["k"], a["out"], a["ws"],
                        ctypes.c_size_t(a["wsb"]), None)


def test_topk_checks(lib):
    assert topk_call(lib, lg=None) == bd.IDX_EINVAL
    assert topk_call(lib, ls=0) == bd.IDX_EINVAL
    assert topk_call(lib, k=0) == bd.IDX_EINVAL
    assert topk_call(lib, B=0) == bd.IDX_EINVAL
    assert topk_call(lib, ls=65537) == bd.IDX_EUNSUPPORTED      # rows beyond the register-held limit
    assert topk_call(lib, ws=None, wsb=512) == bd.IDX_EINVAL
    assert topk_call(lib, ws=FAKE + 16, wsb=512) == bd.IDX_EALIGN


def test_workspace_bytes(lib):
    f = lib.idx_workspace_bytes
    assert f(0, 1, 32, 8192, 1024) == 0 and f(1, 0, 32, 8192, 1024) == 0 and f(1, 1, 0, 8192, 1024) == 0
    assert f(1, 1, 32, -1, 1024) == 0 and f(1, 1, 32, 8192, 0) == 0
    # one block counter per sequence, in 256-byte units
    assert f(1, 1, 32, 8192, 1024) == 256 and f(64, 1, 32, 8192, 1024) == 256 and f(65, 1, 32, 8192, 1024) == 512
    assert all(f(B, 3, 64, 2368, 1024) % 256 == 0 for B in (1, 63, 64, 128, 1000))


def step_call(lib, p=None, **kw):
    """idx_decode_step with valid-looking fake pointers (decode B2/H32/ctx256, k 64)."""
    P = p if p is not None else pool()
    d = dict(k=FAKE, rs=128, g=FAKE, eps=1e-6, pos=FAKE, cs=FAKE, mp=512, sl=FAKE, q=FAKE, qs=FAKE, w=FAKE, pt=FAKE,
             mpp=4, ctx=FAKE, B=2, n_q=1, H=32, D=128, mc=256, lg=FAKE, ls=256, kk=64, out=FAKE, ws=FAKE,
             wsb=lib.idx_workspace_bytes(2, 1, 32, 256, 64))
    d.update(kw)
    return lib.idx_decode_step(ctypes.byref(P), d["k"], d["rs"], d["g"], ctypes.c_float(d["eps"]), d["pos"], d["cs"],
                               d["mp"], d["sl"], d["q"], d["qs"], d["w"], d["pt"], d["mpp"], d["ctx"], d["B"],
                               d["n_q"], d["H"], d["D"], d["mc"], d["lg"], ctypes.c_int64(d["ls"]), d["kk"], d["out"],
                               d["ws"], ctypes.c_size_t(d["wsb"]), None)


def test_decode_step_fused_query(lib):
    assert lib.idx_decode_step_fused(0, 1, 32, 8192) == bd.IDX_EINVAL
    assert lib.idx_decode_step_fused(64, 1, 32, -1) == bd.IDX_EINVAL
    assert lib.idx_decode_step_fused(64, 5, 64, 8192) == bd.IDX_EUNSUPPORTED   # prefill form
    assert lib.idx_decode_step_fused(64, 1, 32, 65537) == bd.IDX_EUNSUPPORTED
    if no_gpu(lib):
        assert lib.idx_decode_step_fused(64, 1, 32, 8192) == bd.IDX_EUNSUPPORTED


def test_decode_step_checks(lib):
    assert step_call(lib, ws=None) == bd.IDX_EINVAL
    assert step_call(lib, wsb=0) == bd.IDX_EINVAL
    assert step_call(lib, wsb=255) == bd.IDX_EINVAL
    assert step_call(lib, ws=FAKE + 2) == bd.IDX_EALIGN
    assert step_call(lib, ws=FAKE + 128) == bd.IDX_EALIGN
    assert step_call(lib, sl=None) == bd.IDX_EINVAL
    assert step_call(lib, rs=64) == bd.IDX_EINVAL
    assert step_call(lib, kk=0) == bd.IDX_EINVAL
    assert step_call(lib, D=64) == bd.IDX_EUNSUPPORTED
    assert step_call(lib, n_q=5, H=64) == bd.IDX_EUNSUPPORTED            # 20 head tiles: not the decode form
    assert step_call(lib, mc=65537, mpp=1 << 11, ls=1 << 17) == bd.IDX_EUNSUPPORTED  # rows past the top-k's
    assert step_call(lib, mc=257) == bd.IDX_EINVAL                       # beyond the page table
    if no_gpu(lib):
        assert step_call(lib) == bd.IDX_EUNSUPPORTED
        # wider shapes pass validation (and run as three kernels on a device)
        assert step_call(lib, H=48) == bd.IDX_EUNSUPPORTED
        assert step_call(lib, mc=16385, mpp=1 << 10, ls=1 << 15) == bd.IDX_EUNSUPPORTED


def test_q_prep_checks(lib):
    f = lambda **kw: lib.idx_q_prep_mxfp4(*[dict(q=FAKE, T=4, H=32, pos=FAKE, cs=FAKE, mp=64, w=FAKE, ws=0.5,
                                                   qp=FAKE, qs=FAKE, wo=FAKE, st=None, **{})[k] if k not in kw
                                            else kw[k] for k in ("q", "T", "H", "pos", "cs", "mp", "w", "ws", "qp",
                                                                 "qs", "wo", "st")])
    assert f(T=-1) == bd.IDX_EINVAL
    assert f(H=0) == bd.IDX_EINVAL
    assert f(H=129) == bd.IDX_EUNSUPPORTED
    assert f(mp=0) == bd.IDX_EINVAL
    assert f(pos=None) == bd.IDX_EINVAL
    assert f(qs=FAKE + 2) == bd.IDX_EALIGN
    assert f(qp=FAKE + 1) == bd.IDX_EALIGN
    assert f(q=FAKE + 8) == bd.IDX_EALIGN   # the bf16 input is read 16 bytes per lane
    if no_gpu(lib):
        assert f() == bd.IDX_EUNSUPPORTED


def test_quant_checks(lib):
    assert lib.idx_q_quant_mxfp4(FAKE, -1, FAKE, FAKE, None) == bd.IDX_EINVAL
    assert lib.idx_q_quant_mxfp4(None, 4, FAKE, FAKE, None) == bd.IDX_EINVAL
    assert lib.idx_q_quant_mxfp4(FAKE, 4, FAKE + 4, FAKE, None) == bd.IDX_EALIGN
    assert lib.idx_q_quant_fp8(FAKE, None, 4, FAKE, FAKE, None) == bd.IDX_EINVAL


def test_valid_calls_report_missing_device(lib):
    """With arguments that pass validation, a machine without gfx950 gets EUNSUPPORTED
    (the caller's signal to fall back), never a launch."""
    if not no_gpu(lib):
        pytest.skip("a GPU is present: fake pointers must not reach a launch")
    assert logits_call(lib) == bd.IDX_EUNSUPPORTED
    assert topk_call(lib) == bd.IDX_EUNSUPPORTED
    assert lib.idx_q_quant_mxfp4(FAKE, 4, FAKE, FAKE, None) == bd.IDX_EUNSUPPORTED
    # zero-sized work still goes through the device gate
    assert lib.idx_device_check() == bd.IDX_EUNSUPPORTED


def test_diag_read_checks(lib):
    out = ctypes.c_void_p(FAKE)
    assert lib.idx_diag_hbm_read(None, 1024, 4, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_hbm_read(FAKE, 1000, 4, out, None) == bd.IDX_EINVAL      # not a multiple of 16
    assert lib.idx_diag_hbm_read(FAKE, 0, 4, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_hbm_read(FAKE, 1024, 0, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_hbm_read(FAKE + 8, 1024, 4, out, None) == bd.IDX_EALIGN
    assert lib.idx_diag_hbm_read(FAKE, 1024, 4, None, None) == bd.IDX_EINVAL


def test_diag_mfma_checks(lib):
    out = ctypes.c_void_p(FAKE)
    assert lib.idx_diag_mfma(2, 1, 1, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_mfma(0, 0, 1, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_mfma(1, 1, -1, out, None) == bd.IDX_EINVAL
    assert lib.idx_diag_mfma(0, 1, 1, None, None) == bd.IDX_EINVAL


def qk_prep_call(lib, p=None, **kw):
    a = dict(q=FAKE, k=FAKE, T=4, H=8, w=FAKE, pos=FAKE, cs=FAKE, max_pos=16, neox=1, g=FAKE, b=FAKE, eps=1e-6,
             slots=FAKE, q8=FAKE, wo=FAKE)
    a.update(kw)
    p = p or pool(kv_format=1, page_stride_bytes=132 * 64)
    return lib.idx_qk_prep_fp8(ctypes.byref(p), a["q"], a["k"], a["T"], a["H"], a["w"], a["pos"], a["cs"],
                               a["max_pos"], a["neox"], a["g"], a["b"], a["eps"], a["slots"], a["q8"], a["wo"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(H=0), bd.IDX_EINVAL),
    (dict(H=129), bd.IDX_EUNSUPPORTED),
    (dict(T=-1), bd.IDX_EINVAL),
    (dict(neox=2), bd.IDX_EINVAL),
    (dict(eps=0.0), bd.IDX_EINVAL),
    (dict(max_pos=0), bd.IDX_EINVAL),
    (dict(k=None), bd.IDX_EINVAL),
    (dict(q8=FAKE + 2), bd.IDX_EALIGN),
    (dict(q=FAKE + 8), bd.IDX_EALIGN),               # the bf16 queries are read 16 bytes per lane
    (dict(T=(1 << 26) // 9 + 1), bd.IDX_EINVAL),   # the grid would pass 2^32 work-items
])
def test_qk_prep_checks(lib, kw, want):
    assert qk_prep_call(lib, **kw) == want


def test_qk_prep_needs_an_fp8_pool(lib):
    assert qk_prep_call(lib, p=pool()) == bd.IDX_EINVAL



def cand_call(lib, p=None, **kw):
    """idx_logits_candidates with valid-looking fake pointers (B2, H4, 4 blocks of 64)."""
    a = dict(q=FAKE, qs=FAKE, w=FAKE, pt=FAKE, maxp=4, ctx=FAKE, B=2, n_q=1, H=4, D=128, cand=FAKE, nc=4,
             logits=FAKE, lstride=256)
    a.update(kw)
    p = p or pool()
    return lib.idx_logits_candidates(ctypes.byref(p), a["q"], a["qs"], a["w"], a["pt"], a["maxp"], a["ctx"], a["B"],
                                     a["n_q"], a["H"], a["D"], a["cand"], a["nc"], a["logits"],
                                     ctypes.c_int64(a["lstride"]), None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=64), bd.IDX_EUNSUPPORTED),
    (dict(H=0), bd.IDX_EINVAL),
    (dict(nc=-1), bd.IDX_EINVAL),
    (dict(cand=None), bd.IDX_EINVAL),
    (dict(lstride=255), bd.IDX_EINVAL),                       # fewer than n_cand * P cells
    (dict(nc=1025, lstride=1 << 20), bd.IDX_EUNSUPPORTED),   # more than 65536 cells
    (dict(maxp=1 << 25), bd.IDX_EINVAL),                      # token ids past int32
    (dict(qs=None), bd.IDX_EINVAL),
    (dict(q=FAKE + 8), bd.IDX_EALIGN),
])
def test_candidate_argument_checks(lib, kw, want):
    assert cand_call(lib, **kw) == want


def test_topk_candidate_checks(lib):
    f = lib.idx_topk_candidates
    assert f(None, 256, FAKE, 4, 64, 2, 1, 64, FAKE, None) == bd.IDX_EINVAL
    assert f(FAKE, 256, None, 4, 64, 2, 1, 64, FAKE, None) == bd.IDX_EINVAL
    assert f(FAKE, 255, FAKE, 4, 64, 2, 1, 64, FAKE, None) == bd.IDX_EINVAL
    assert f(FAKE, 256, FAKE, 4, 48, 2, 1, 64, FAKE, None) == bd.IDX_EUNSUPPORTED
    assert f(FAKE, 256, FAKE, 4, 64, 2, 1, 0, FAKE, None) == bd.IDX_EINVAL
    assert f(FAKE, 1 << 20, FAKE, 1025, 64, 2, 1, 64, FAKE, None) == bd.IDX_EUNSUPPORTED
    if no_gpu(lib):
        assert cand_call(lib) == bd.IDX_EUNSUPPORTED
        assert f(FAKE, 256, FAKE, 4, 64, 2, 1, 64, FAKE, None) == bd.IDX_EUNSUPPORTED
