"""Pins for the oracle's paged MQA logits with the causal/length mask.

Anchors: an independent exact computation (E2M1 from the literal spec table, products
as integers times powers of two, weights as exact rationals); closed forms (one-hot q
and k, w = e_h gives ReLU(d_h), non-negative w gives non-negative logits); invariance
under physical-page permutation, pool offset and page stride; the valid-length rule
for decode, speculative verification and prefill; and a pure-Python brute force over
the whole tiny-decode workload.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _indep as ind

TWO_E2M1 = [int(2 * m) for m in ind.E2M1_MAG]  # {0,1,2,3,4,6,8,12}: integers


def rand_mxfp4_case(rng, B, n_q, H, ctx, P, extra_pages=3, offset=0, gap=0):
    ctx = np.asarray(ctx, np.int32)
    need = [(int(c) + P - 1) // P for c in ctx]
    num_pages = sum(need) + extra_pages
    stride = 68 * P + gap
    pool = rng.integers(0, 256, offset + num_pages * stride, dtype=np.uint8)
    pids = rng.permutation(num_pages)
    pt = np.full((B, max(need)), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        pt[b, :n] = pids[pos:pos + n]
        pos += n
    for p in range(num_pages):  # scales in a moderate range so products stay well inside fp64
        base = offset + p * stride + 64 * P
        pool[base: base + 4 * P] = rng.integers(118, 136, 4 * P)
    q = rng.integers(0, 256, (B, n_q, H, 64), dtype=np.uint8)
    qs = rng.integers(118, 136, (B, n_q, H, 4), dtype=np.uint8)
    w = (rng.standard_normal((B, n_q, H)) / np.sqrt(H)).astype(np.float32)
    return dict(pool=pool, offset=offset, stride=stride, num_pages=num_pages, P=P, q=q, qs=qs, w=w, pt=pt, ctx=ctx,
                B=B, n_q=n_q, H=H)


def run_oracle(c, rows=None, out_stride=None):
    out_stride = out_stride or int(c["ctx"].max())
    return oracle.logits_paged(c["pool"], c["offset"], c["stride"], c["num_pages"], c["P"], oracle.FMT_MXFP4, c["q"],
                               c["qs"], c["w"], c["pt"], c["ctx"], c["B"], c["n_q"], c["H"], out_stride, rows)


def exact_dot(qb, qsb, kb, ksb):
    """q.k exactly: sum over 32-blocks of 2^(Xq + Xk - 2) * sum_i (2 q_i)(2 k_i)."""
    qn, kn = ind.unpack_nibbles(bytes(qb)), ind.unpack_nibbles(bytes(kb))
    total = Fraction(0)
    for blk in range(4):
        acc = 0
        for i in range(32 * blk, 32 * blk + 32):
            a, b = qn[i], kn[i]
            va = TWO_E2M1[a & 7] * (-1 if a & 8 else 1)
            vb = TWO_E2M1[b & 7] * (-1 if b & 8 else 1)
            acc += va * vb
        total += Fraction(acc) * Fraction(2) ** (int(qsb[blk]) - 127 + int(ksb[blk]) - 127 - 2)
    return total


def exact_logit(c, r, s):
    b, j = divmod(r, c["n_q"])
    pid = int(c["pt"][b, s // c["P"]])
    row = s % c["P"]
    base = c["offset"] + pid * c["stride"]
    kb = c["pool"][base + row * 64: base + row * 64 + 64]
    ksb = c["pool"][base + 64 * c["P"] + row * 4: base + 64 * c["P"] + row * 4 + 4]
    tot = Fraction(0)
    for h in range(c["H"]):
        d = exact_dot(c["q"][b, j, h], c["qs"][b, j, h], kb, ksb)
        tot += Fraction(float(c["w"][b, j, h])) * max(d, Fraction(0))
    return tot


def test_matches_exact_integer_computation():
    rng = np.random.default_rng(20)
    c = rand_mxfp4_case(rng, B=2, n_q=2, H=5, ctx=[70, 33], P=32)
    out = run_oracle(c)
    for r in range(4):
        b, j = divmod(r, 2)
        n = min(max(int(c["ctx"][b]) - 2 + 1 + j, 0), int(c["ctx"][b]))
        for s in range(0, n, 3):
            ex = exact_logit(c, r, s)
            assert abs(Fraction(out[r, s]) - ex) <= Fraction(1, 10 ** 12) * (abs(ex) + 1), (r, s)


def test_valid_length_rule_and_mask():
    rng = np.random.default_rng(21)
    c = rand_mxfp4_case(rng, B=3, n_q=3, H=2, ctx=[10, 2, 40], P=16)
    out = run_oracle(c, out_stride=48)
    want = {0: 8, 1: 9, 2: 10, 3: 0, 4: 1, 5: 2, 6: 38, 7: 39, 8: 40}
    for r, n in want.items():
        assert oracle.valid_len(c["ctx"], 3, r) == n
        assert np.all(np.isfinite(out[r, :n])) and np.all(np.isnan(out[r, n:])), r


def test_prefill_is_causal():
    rng = np.random.default_rng(22)
    c = rand_mxfp4_case(rng, B=1, n_q=50, H=3, ctx=[50], P=16)
    out = run_oracle(c)
    for j in range(50):
        assert np.all(np.isfinite(out[j, :j + 1])) and np.all(np.isnan(out[j, j + 1:]))


def _one_hot_case(qi, ki, qv_code, kv_code, qscale=127, kscale=127):
    B, n_q, H, P = 1, 1, 1, 16
    pool = np.zeros(68 * P, np.uint8)
    pool[64 * P: 64 * P + 4] = kscale
    pool[ki // 2] = kv_code << (4 * (ki % 2))
    q = np.zeros((1, 1, 1, 64), np.uint8)
    q[0, 0, 0, qi // 2] = qv_code << (4 * (qi % 2))
    qs = np.full((1, 1, 1, 4), qscale, np.uint8)
    w = np.ones((1, 1, 1), np.float32)
    return oracle.logits_paged(pool, 0, 68 * P, 1, P, oracle.FMT_MXFP4, q, qs, w, np.zeros((1, 1), np.int32),
                               np.array([1], np.int32), B, n_q, H, 1)[0, 0]


def test_one_hot_closed_forms():
    mags = ind.GOLDEN["e2m1_magnitudes"]["value"]
    for i in (0, 1, 31, 32, 77, 127):
        for a in range(1, 8):
            for b in (1, 5, 7):
                assert _one_hot_case(i, i, a, b) == mags[a] * mags[b]
                assert _one_hot_case(i, i, a | 8, b) == 0.0          # negative dot -> ReLU -> 0
        assert _one_hot_case(i, (i + 1) % 128, 7, 7) == 0.0          # different dims do not meet
    # scales: block scale bytes multiply as powers of two
    assert _one_hot_case(5, 5, 2, 2, qscale=130, kscale=120) == 1.0 * 2.0 ** (3 - 7)


def test_weights_select_heads_and_sign():
    rng = np.random.default_rng(23)
    c = rand_mxfp4_case(rng, B=1, n_q=1, H=4, ctx=[64], P=32)
    for h in range(4):
        cc = dict(c)
        cc["w"] = np.zeros_like(c["w"])
        cc["w"][0, 0, h] = 1.0
        out = run_oracle(cc)[0]
        for s in range(0, 64, 7):
            ex = exact_logit(cc, 0, s)
            assert Fraction(out[s]) == ex and out[s] >= 0
    cc = dict(c)
    cc["w"] = np.abs(c["w"])
    assert np.all(run_oracle(cc)[0] >= 0)


def test_page_permutation_offset_and_stride_invariance():
    rng = np.random.default_rng(24)
    c = rand_mxfp4_case(rng, B=2, n_q=1, H=3, ctx=[100, 64], P=32)
    base = run_oracle(c)
    # move every physical page to a new slot, with a pool offset and a larger stride
    perm = rng.permutation(c["num_pages"])
    new_stride, new_off = c["stride"] + 512, 768
    pool2 = np.full(new_off + c["num_pages"] * new_stride, 0x5A, np.uint8)
    for old in range(c["num_pages"]):
        src = c["pool"][old * c["stride"]:(old + 1) * c["stride"]]
        dst = new_off + perm[old] * new_stride
        pool2[dst: dst + c["stride"]] = src
    pt2 = np.where(c["pt"] >= 0, perm[np.maximum(c["pt"], 0)], -1).astype(np.int32)
    c2 = dict(c, pool=pool2, offset=new_off, stride=new_stride, pt=pt2)
    np.testing.assert_array_equal(run_oracle(c2), base)
    # and a wrong page map changes the answer (sensitivity)
    pt3 = pt2.copy()
    pt3[0, 0], pt3[0, 1] = pt2[0, 1], pt2[0, 0]
    c3 = dict(c2, pt=pt3)
    assert not np.array_equal(run_oracle(c3)[~np.isnan(base)], base[~np.isnan(base)])


def test_row_subset_equals_full():
    rng = np.random.default_rng(25)
    c = rand_mxfp4_case(rng, B=3, n_q=2, H=2, ctx=[20, 30, 40], P=16)
    full = run_oracle(c)
    rows = np.array([5, 0, 3], np.int64)
    np.testing.assert_array_equal(run_oracle(c, rows=rows), full[rows])


@pytest.mark.slow
def test_tiny_decode_brute_force():
    """Every valid cell of the tiny decode workload, by pure-Python loops over bytes."""
    W = wl.make_workload(0)
    stride = W.page_stride_bytes
    pool = np.zeros(W.pool_bytes, np.uint8)
    oracle.k_store(pool, W.offset_bytes, stride, W.num_pages, W.page_size, oracle.FMT_MXFP4, W.k_rows, W.gamma, W.eps,
                   W.positions, W.cos_sin, W.slots)
    q, qs = oracle.q_quant_mxfp4(W.q_rows)
    c = dict(pool=pool, offset=W.offset_bytes, stride=stride, num_pages=W.num_pages, P=W.page_size, q=q, qs=qs, w=W.w,
             pt=W.page_table, ctx=W.ctx, B=W.B, n_q=W.n_q, H=W.H)
    out = run_oracle(c)
    for r in range(W.rows):
        for s in range(W.valid_len(r)):
            ex = exact_logit(c, r, s)
            assert abs(Fraction(out[r, s]) - ex) <= Fraction(1, 10 ** 12) * (abs(ex) + 1)


def test_fp8_logits_exact():
    rng = np.random.default_rng(26)
    B, n_q, H, P = 1, 2, 3, 16
    ctx = np.array([30], np.int32)
    pool = np.zeros(2 * 132 * P, np.uint8)
    codes = rng.integers(0, 0x7F, (2 * P, 128)).astype(np.uint8) | (rng.integers(0, 2, (2 * P, 128)) << 7).astype(np.uint8)
    sks = (rng.uniform(0.5, 2.0, 2 * P)).astype(np.float32)
    for t in range(2 * P):
        p, r = divmod(t, P)
        pool[p * 132 * P + r * 128: p * 132 * P + r * 128 + 128] = codes[t]
        pool[p * 132 * P + 128 * P + 4 * r: p * 132 * P + 128 * P + 4 * r + 4] = np.frombuffer(sks[t].tobytes(), np.uint8)
    q8 = rng.integers(0, 0x7F, (B, n_q, H, 128)).astype(np.uint8)
    w = rng.standard_normal((B, n_q, H)).astype(np.float32)
    pt = np.array([[1, 0]], np.int32)
    out = oracle.logits_paged(pool, 0, 132 * P, 2, P, oracle.FMT_FP8, q8, None, w, pt, ctx, B, n_q, H, 30)
    for r in range(2):
        for s in range(oracle.valid_len(ctx, n_q, r)):
            t = int(pt[0, s // P]) * P + s % P
            tot = Fraction(0)
            for h in range(H):
                d = sum(ind.e4m3_value(int(q8[0, r, h, i])) * ind.e4m3_value(int(codes[t, i])) for i in range(128))
                d *= Fraction(float(sks[t]))
                tot += Fraction(float(w[0, r, h])) * max(d, Fraction(0))
            assert abs(Fraction(out[r, s]) - tot) <= Fraction(1, 10 ** 12) * (abs(tot) + 1)


# ----------------------------------------------------------------------------------------
# The unquantised scorer (oracle.logits_exact): the method on fp64 rows with no MXFP4 or
# e4m3 rounding, used as the reference of the same-run precision comparison.

def _dequant_mxfp4(nibble_bytes, scale_bytes):
    """fp64 values of packed MXFP4 vectors from the spec table (independent of the oracle):
    [..., 64] nibble bytes + [..., 4] E8M0 bytes -> [..., 128]."""
    lut = np.array([float(v) for v in ind.E2M1_VALUES], np.float64)
    nb = np.asarray(nibble_bytes, np.uint8)
    codes = np.stack([nb & 15, nb >> 4], axis=-1).reshape(nb.shape[:-1] + (128,))
    scale = np.ldexp(1.0, np.asarray(scale_bytes, np.int64) - 127)             # [..., 4]
    return lut[codes] * np.repeat(scale, 32, axis=-1)


def test_logits_exact_equals_paged_on_representable_rows():
    """On rows that MXFP4 represents exactly, the unquantised scorer fed the dequantised
    rows must give the packed scorer's logits bit for bit (every product and block sum is
    exact in fp64, so no rounding order can separate them), masked cells included."""
    rng = np.random.default_rng(27)
    for (B, n_q, H, ctx, P) in ((2, 1, 4, [70, 33], 32), (1, 5, 3, [40], 16), (3, 2, 2, [16, 1, 50], 16)):
        c = rand_mxfp4_case(rng, B=B, n_q=n_q, H=H, ctx=ctx, P=P)
        S = int(c["ctx"].max())
        k_rows = np.zeros((B, S, 128), np.float64)
        for b in range(B):
            for s in range(int(c["ctx"][b])):
                base = c["offset"] + int(c["pt"][b, s // P]) * c["stride"]
                row = s % P
                k_rows[b, s] = _dequant_mxfp4(c["pool"][base + 64 * row: base + 64 * row + 64],
                                              c["pool"][base + 64 * P + 4 * row: base + 64 * P + 4 * row + 4])
        q_rows = _dequant_mxfp4(c["q"], c["qs"]).reshape(B * n_q, H, 128)
        rows = np.arange(B * n_q, dtype=np.int64)
        got = oracle.logits_exact(q_rows, c["w"].reshape(-1), k_rows, c["ctx"], n_q, H, S, rows)
        want = run_oracle(c, out_stride=S)
        np.testing.assert_array_equal(got, want)


def test_logits_exact_integer_brute_force():
    """Small-integer rows and power-of-two weights keep every step exact; the expected
    logits come from Python integers and Fractions cell by cell (the valid-length rule
    included: masked cells are NaN)."""
    rng = np.random.default_rng(28)
    B, n_q, H, S = 2, 3, 5, 9
    ctx = np.array([9, 4], np.int32)
    q_rows = rng.integers(-3, 4, (B * n_q, H, 128)).astype(np.float64)
    k_rows = rng.integers(-3, 4, (B, S, 128)).astype(np.float64)
    w = np.ldexp(1.0, rng.integers(-4, 4, B * n_q * H)) * rng.choice([-1.0, 1.0], B * n_q * H)
    w = w.astype(np.float32)
    rows = np.arange(B * n_q, dtype=np.int64)
    got = oracle.logits_exact(q_rows, w, k_rows, ctx, n_q, H, S, rows)
    for r in range(B * n_q):
        b, j = divmod(r, n_q)
        n = max(0, min(int(ctx[b]) - n_q + 1 + j, int(ctx[b])))
        for s in range(S):
            if s >= n:
                assert np.isnan(got[r, s]), (r, s)
                continue
            tot = Fraction(0)
            for h in range(H):
                d = sum(int(q_rows[r, h, i]) * int(k_rows[b, s, i]) for i in range(128))
                tot += Fraction(float(w[r * H + h])) * max(d, 0)
            assert Fraction(got[r, s]) == tot, (r, s)


def test_logits_exact_one_hot_and_parallel_closed_forms():
    """One-hot rows meet only on equal dims; a query head parallel to the key scores
    c * |k|^2 through the ReLU (zero for c < 0); the weights pick and scale heads."""
    H = 3
    k = np.zeros((1, 4, 128), np.float64)
    for s, i in enumerate((0, 31, 64, 127)):
        k[0, s, i] = 2.0 ** s
    q = np.zeros((1, H, 128), np.float64)
    q[0, 0, 31] = 3.0        # meets token 1 only
    q[0, 1, 127] = -5.0      # meets token 3 with a negative dot: ReLU gives 0
    q[0, 2, 64] = 0.5        # meets token 2
    w = np.array([1.0, 7.0, 4.0], np.float32)
    got = oracle.logits_exact(q, w, k, np.array([4], np.int32), 1, H, 4, np.array([0], np.int64))[0]
    np.testing.assert_array_equal(got, [0.0, 1.0 * 3.0 * 2.0, 4.0 * 0.5 * 4.0, 0.0])
    rng = np.random.default_rng(29)
    kv = rng.integers(-4, 5, 128).astype(np.float64)
    norm2 = float(kv @ kv)
    k2 = kv.reshape(1, 1, 128)
    coef = np.array([2.0, -1.0, 0.25, 3.0])
    q2 = (coef[:, None] * kv[None, :]).reshape(1, 4, 128)
    w2 = np.array([1.0, 100.0, -2.0, 0.5], np.float32)
    got2 = oracle.logits_exact(q2, w2, k2, np.array([1], np.int32), 1, 4, 1, np.array([0], np.int64))[0, 0]
    assert got2 == (1.0 * 2.0 + 0.0 - 2.0 * 0.25 + 0.5 * 3.0) * norm2
