"""Pins of the oracle's MXFP4 Q preparation (rotation, packing, weight fold).

Rotations whose factors are exact (identity, quarter turn, half turn) reduce the op to
the plain Q packing of a permuted / negated vector, which pins the pairing (i, i+32), the
signs and the pass-through of dims 64..127; a general angle is checked against the exact
rotation within the MXFP4 error bound; the weight fold is pinned with exact factors."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import workloads as wl


def qvecs(rng, T, H):
    x = rng.standard_normal((T, H, 128)).astype(np.float32) * rng.uniform(0.1, 30.0, (T, H, 1)).astype(np.float32)
    x[x == 0] = 1.0  # no signed zeros: their sign may legitimately flip under a rotation
    return wl.f32_to_bf16_bits(x)


def table(c, n, rows=4):
    cs = np.zeros((rows, 64), np.float32)
    cs[:, :32] = c
    cs[:, 32:] = n
    return cs


def bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def neg(b):
    return (b ^ np.uint16(0x8000)).astype(np.uint16)


@pytest.mark.parametrize("T,H", [(3, 4), (1, 1), (5, 20)])
def test_identity_rotation_is_plain_packing(T, H):
    rng = np.random.default_rng(T * 10 + H)
    q = qvecs(rng, T, H)
    p, s, _ = oracle.q_prep_mxfp4(q, np.zeros(T, np.int32), table(1.0, 0.0), np.ones((T, H), np.float32), 1.0)
    p0, s0 = oracle.q_quant_mxfp4(q)
    assert np.array_equal(p, p0.reshape(p.shape)) and np.array_equal(s, s0.reshape(s.shape))


def test_quarter_turn_swaps_and_negates_the_rope_halves():
    """cos 0, sin 1: z_i = -x_{i+32}, z_{i+32} = x_i for i < 32, z_i = x_i for i >= 64."""
    rng = np.random.default_rng(7)
    q = qvecs(rng, 4, 8)
    p, s, _ = oracle.q_prep_mxfp4(q, np.full(4, 2, np.int32), table(0.0, 1.0), np.ones((4, 8), np.float32), 1.0)
    x2 = np.concatenate([neg(q[..., 32:64]), q[..., 0:32], q[..., 64:]], axis=-1)
    p0, s0 = oracle.q_quant_mxfp4(x2)
    assert np.array_equal(p, p0.reshape(p.shape)) and np.array_equal(s, s0.reshape(s.shape))


def test_half_turn_negates_the_rope_dims_only():
    rng = np.random.default_rng(8)
    q = qvecs(rng, 2, 16)
    p, s, _ = oracle.q_prep_mxfp4(q, np.full(2, 1, np.int32), table(-1.0, 0.0), np.ones((2, 16), np.float32), 1.0)
    x2 = np.concatenate([neg(q[..., :64]), q[..., 64:]], axis=-1)
    p0, s0 = oracle.q_quant_mxfp4(x2)
    assert np.array_equal(p, p0.reshape(p.shape)) and np.array_equal(s, s0.reshape(s.shape))


def test_position_outside_the_table_leaves_the_vector_unrotated():
    rng = np.random.default_rng(9)
    q = qvecs(rng, 3, 4)
    cs = wl.rope_cos_sin(16)
    p, s, _ = oracle.q_prep_mxfp4(q, np.array([-1, 16, 1 << 30], np.int32), cs, np.ones((3, 4), np.float32), 1.0)
    p0, s0 = oracle.q_quant_mxfp4(q)
    assert np.array_equal(p, p0.reshape(p.shape)) and np.array_equal(s, s0.reshape(s.shape))


def test_general_angle_within_the_mxfp4_bound():
    """Dequantised output vs the exact rotation: within 2^(X+1) per element, X the
    block's scale exponent (half a grid step, or the clip of values past 6 * 2^X)."""
    rng = np.random.default_rng(10)
    T, H = 6, 8
    q = qvecs(rng, T, H)
    cs = wl.rope_cos_sin(4096)
    pos = rng.integers(0, 4096, T).astype(np.int32)
    p, s, _ = oracle.q_prep_mxfp4(q, pos, cs, np.ones((T, H), np.float32), 1.0)
    x = bits_to_f32(q).astype(np.float64)
    c = cs[pos, :32].astype(np.float64)[:, None, :]
    n = cs[pos, 32:].astype(np.float64)[:, None, :]
    z = x.copy()
    z[..., :32] = x[..., :32] * c - x[..., 32:64] * n
    z[..., 32:64] = x[..., 32:64] * c + x[..., :32] * n
    lo, hi = p & 0x0F, p >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(T, H, 128)
    mag = np.array([oracle.e2m1_decode(int(v)) for v in range(16)])
    X = s.astype(np.int64) - 127
    deq = mag[codes] * np.exp2(np.repeat(X, 32, axis=-1))
    bound = np.exp2(np.repeat(X + 1, 32, axis=-1))
    assert np.all(np.abs(deq - z) <= bound)
    # and the rotation moved something: not the unrotated packing
    p0, _ = oracle.q_quant_mxfp4(q)
    assert not np.array_equal(p, p0.reshape(p.shape))


def test_weight_fold_with_exact_factors():
    rng = np.random.default_rng(11)
    q = qvecs(rng, 2, 4)
    w = rng.standard_normal((2, 4)).astype(np.float32)
    cs = wl.rope_cos_sin(8)
    pos = np.array([1, 2], np.int32)
    assert np.array_equal(oracle.q_prep_mxfp4(q, pos, cs, w, 1.0)[2], w)
    assert np.array_equal(oracle.q_prep_mxfp4(q, pos, cs, w, 2.0 ** -5)[2], w / np.float32(32.0))
    assert np.all(oracle.q_prep_mxfp4(q, pos, cs, w, 0.0)[2] == 0.0)
    # the fold rounds once: 1/sqrt(128) * 1/sqrt(32) = 1/64 exactly, whatever the order
    assert np.array_equal(oracle.q_prep_mxfp4(q, pos, cs, w, 1.0 / 64.0)[2], w / np.float32(64.0))
