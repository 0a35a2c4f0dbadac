"""Pins of the oracle's FP8 QK preparation (LayerNorm on k, NeoX or interleaved RoPE on q
and k, FP8 k to the pages, per-vector FP8 q with its scale folded into the weights,
skipped rows zeroed).

The pins tie it to independently pinned parts or to closed forms:
  - a zero-mean row with beta = 0 is the K store's RMSNorm row (LayerNorm = RMSNorm);
  - shifting a row by a constant (exactly) leaves its LayerNorm bytes unchanged;
  - gamma = 0 stores beta itself, quantised as a plain FP8 vector;
  - an identity rotation leaves Q as the plain per-vector FP8 quantisation and fold;
  - a half or quarter turn permutes and negates codes of the identity case (both
    layouts, both q and k), which pins the pairing of each layout;
  - a general angle stays within the e4m3 rounding bound of an fp64 LayerNorm + RoPE
    written here with numpy;
  - rows with a padding slot, a slot outside the pool or a position outside the table
    store nothing and get zero codes and weights."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import workloads as wl

P = 16
NPAGES = 8
STRIDE = 132 * P


def bf(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def table(c, n, rows=4):
    cs = np.zeros((rows, 64), np.float32)
    cs[:, :32] = c
    cs[:, 32:] = n
    return cs


def run(q, k, w, pos, cs, neox, gamma, beta, slots, eps=1e-6):
    pool = np.full(NPAGES * STRIDE, 0xA5, np.uint8)
    q8, wo = oracle.qk_prep_fp8(pool, 0, STRIDE, NPAGES, P, q, k, w, pos, cs, neox, gamma, beta, eps, slots)
    return pool, q8, wo


def k_bytes(pool, slot):
    page = pool[(slot // P) * STRIDE: (slot // P + 1) * STRIDE]
    r = slot % P
    return page[r * 128: r * 128 + 128].copy(), page[P * 128 + r * 4: P * 128 + r * 4 + 4].view(np.float32)[0]


def inputs(rng, T, H, nonzero=True):
    q = rng.standard_normal((T, H, 128)).astype(np.float32) * rng.uniform(0.1, 20.0, (T, H, 1)).astype(np.float32)
    k = rng.standard_normal((T, 128)).astype(np.float32) * 3.0
    if nonzero:
        q[q == 0] = 1.0
        k[k == 0] = 1.0
    w = rng.standard_normal((T, H)).astype(np.float32)
    return bf(q), bf(k), w


def test_zero_mean_row_with_zero_beta_is_the_rmsnorm_k_store():
    rng = np.random.default_rng(1)
    T, H = 5, 2
    v = rng.standard_normal((T, 64)).astype(np.float32)
    v[v == 0] = 0.5
    k = bf(np.concatenate([v, -v], axis=1))          # fold sums are exactly zero
    q, _, w = inputs(rng, T, H)
    gamma = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    cs = wl.rope_cos_sin(64)
    pos = rng.integers(0, 64, T).astype(np.int32)
    slots = np.array([3, 17, 40, 64 + 5, 127], np.int64)
    pool, _, _ = run(q, k, w, pos, cs, True, gamma, np.zeros(128, np.float32), slots, eps=1e-5)
    ref = np.full(NPAGES * STRIDE, 0xA5, np.uint8)
    oracle.k_store(ref, 0, STRIDE, NPAGES, P, oracle.FMT_FP8, k, gamma, 1e-5, pos, cs, slots)
    assert np.array_equal(pool, ref)


def test_layernorm_is_shift_invariant_on_exact_inputs():
    rng = np.random.default_rng(2)
    T, H = 4, 1
    base = rng.integers(-20, 20, (T, 128)).astype(np.float32)
    base[base == 0] = 1.0
    gamma = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    beta = rng.uniform(-0.5, 0.5, 128).astype(np.float32)
    q, _, w = inputs(rng, T, H)
    cs = wl.rope_cos_sin(16)
    pos = np.arange(T, dtype=np.int32)
    slots = np.arange(T, dtype=np.int64) * 7
    a, _, _ = run(q, bf(base), w, pos, cs, False, gamma, beta, slots)
    b, _, _ = run(q, bf(base + 8.0), w, pos, cs, False, gamma, beta, slots)   # still exact in bf16
    assert np.array_equal(a, b)


def test_zero_gamma_stores_beta():
    rng = np.random.default_rng(3)
    T, H = 3, 1
    q, k, w = inputs(rng, T, H)
    beta = rng.standard_normal(128).astype(np.float32)
    beta_bf = bf(beta)
    beta_exact = f32(beta_bf)                        # a bf16-exact beta, so the expected vector is exact
    pos = np.zeros(T, np.int32)
    slots = np.array([0, 33, 90], np.int64)
    pool, _, _ = run(q, k, w, pos, table(1.0, 0.0), True, np.zeros(128, np.float32), beta_exact, slots)
    codes, wo = oracle.q_quant_fp8(beta_bf[None, :], np.ones(1, np.float32))
    for s in slots:
        c, sk = k_bytes(pool, int(s))
        assert np.array_equal(c, codes[0]) and sk == wo[0]


@pytest.mark.parametrize("neox", [True, False])
def test_identity_rotation_q_is_plain_fp8_quant_and_fold(neox):
    rng = np.random.default_rng(4)
    T, H = 4, 6
    q, k, w = inputs(rng, T, H)
    pos = np.full(T, 2, np.int32)
    _, q8, wo = run(q, k, w, pos, table(1.0, 0.0), neox, np.ones(128, np.float32), np.zeros(128, np.float32),
                    np.arange(T, dtype=np.int64))
    r8, rw = oracle.q_quant_fp8(q, w)
    assert np.array_equal(q8, r8) and np.array_equal(wo, rw)


def pairs(neox):
    i = np.arange(32)
    return (i, i + 32) if neox else (2 * i, 2 * i + 1)


@pytest.mark.parametrize("neox", [True, False])
def test_half_and_quarter_turns_permute_and_negate_codes(neox):
    rng = np.random.default_rng(5 + neox)
    T, H = 4, 3
    q, k, w = inputs(rng, T, H)
    gamma = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    beta = rng.uniform(-0.3, 0.3, 128).astype(np.float32)
    pos = np.full(T, 1, np.int32)
    slots = np.array([1, 20, 45, 100], np.int64)
    args = (gamma, beta, slots)
    p0, q0, w0 = run(q, k, w, pos, table(1.0, 0.0), neox, *args)
    ph, qh, wh = run(q, k, w, pos, table(-1.0, 0.0), neox, *args)
    pq, qq, wq = run(q, k, w, pos, table(0.0, 1.0), neox, *args)
    a, b = pairs(neox)
    # half turn: dims 0..63 negated (sign bit), everything else equal
    exp_q = q0.copy()
    exp_q[..., :64] ^= 0x80
    assert np.array_equal(qh, exp_q) and np.array_equal(wh, w0)
    # quarter turn: first' = -second, second' = first
    exp_q = q0.copy()
    exp_q[..., a] = q0[..., b] ^ 0x80
    exp_q[..., b] = q0[..., a]
    assert np.array_equal(qq, exp_q) and np.array_equal(wq, w0)
    for s in slots:
        c0, s0 = k_bytes(p0, int(s))
        ch, sh = k_bytes(ph, int(s))
        cq, sq = k_bytes(pq, int(s))
        e = c0.copy()
        e[:64] ^= 0x80
        assert np.array_equal(ch, e) and sh == s0
        e = c0.copy()
        e[a] = c0[b] ^ 0x80
        e[b] = c0[a]
        assert np.array_equal(cq, e) and sq == s0


def e4m3_value(c):
    return np.array([oracle.e4m3_decode(int(x)) for x in np.ravel(c)]).reshape(np.shape(c))


def rope_np(y, c, n, neox):
    z = y.copy()
    a, b = pairs(neox)
    z[..., a] = y[..., a] * c - y[..., b] * n
    z[..., b] = y[..., b] * c + y[..., a] * n
    return z


@pytest.mark.parametrize("neox", [True, False])
def test_general_angle_within_the_e4m3_bound(neox):
    """Dequantised outputs against numpy fp64 LayerNorm + RoPE: within half an e4m3 step
    at each element's magnitude (2^-4 relative) or half the subnormal step."""
    rng = np.random.default_rng(7 + neox)
    T, H = 6, 4
    q, k, w = inputs(rng, T, H)
    gamma = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    beta = rng.uniform(-0.3, 0.3, 128).astype(np.float32)
    cs = wl.rope_cos_sin(4096)
    pos = rng.integers(0, 4096, T).astype(np.int32)
    slots = np.arange(T, dtype=np.int64) * 11
    pool, q8, wo = run(q, k, w, pos, cs, neox, gamma, beta, slots, eps=1e-6)
    c = cs[pos, :32].astype(np.float64)
    n = cs[pos, 32:].astype(np.float64)
    x = f32(k).astype(np.float64)
    d = x - x.mean(axis=1, keepdims=True)
    y = d / np.sqrt((d * d).mean(axis=1, keepdims=True) + 1e-6) * gamma + beta
    zk = rope_np(y, c, n, neox)
    for t, s in enumerate(slots):
        codes, sk = k_bytes(pool, int(s))
        deq = e4m3_value(codes) * np.float64(sk)
        assert np.all(np.abs(deq - zk[t]) <= np.abs(zk[t]) * 2.0 ** -4 + np.float64(sk) * 2.0 ** -10 + 1e-12)
    zq = rope_np(f32(q).astype(np.float64), c[:, None, :], n[:, None, :], neox)
    sq = np.abs(zq).max(axis=2) / 448.0
    deq = e4m3_value(q8) * sq[..., None]
    assert np.all(np.abs(deq - zq) <= np.abs(zq) * 2.0 ** -4 + sq[..., None] * 2.0 ** -10 * 1.0001 + 1e-12)
    assert np.allclose(wo, w * sq.astype(np.float32), rtol=1e-6)


def test_skipped_rows_store_nothing_and_zero_q():
    rng = np.random.default_rng(9)
    T, H = 5, 3
    q, k, w = inputs(rng, T, H)
    cs = wl.rope_cos_sin(8)
    pos = np.array([1, 2, 9, -1, 3], np.int32)       # rows 2 and 3: position outside the table
    slots = np.array([-1, NPAGES * P, 5, 6, 7], np.int64)  # row 0: padding, row 1: outside the pool
    pool, q8, wo = run(q, k, w, pos, cs, True, np.ones(128, np.float32), np.zeros(128, np.float32), slots)
    for t in range(4):
        assert np.all(q8[t] == 0) and np.all(wo[t] == 0)
    assert np.any(q8[4] != 0) and np.any(wo[4] != 0)
    untouched = np.full(NPAGES * STRIDE, 0xA5, np.uint8)
    written = k_bytes(pool, 7)[0]
    assert not np.array_equal(written, untouched[:128])
    pool2 = pool.copy()
    pool2[0: STRIDE] = 0xA5                          # slot 7 lives in page 0: clear it, the rest is untouched
    assert np.array_equal(pool2, untouched)
