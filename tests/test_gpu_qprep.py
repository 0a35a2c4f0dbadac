"""GPU parity: MXFP4 Q preparation (rotation, packing, weight fold) against the oracle,
bit for bit: packed nibbles, scale bytes and folded weights."""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_idx_amd import binding as bd
from sparse_attention_indexer_idx_amd import workloads as wl
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def run(q_bits, pos, cs, w, w_scale):
    torch = G.torch_cuda()
    T, H = q_bits.shape[0], q_bits.shape[1]
    qp = torch.full((T, H, 64), 0xA5, dtype=torch.uint8, device="cuda")
    qs = torch.full((T, H, 4), 0xA5, dtype=torch.uint8, device="cuda")
    wo = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    bd.idx_q_prep_mxfp4(G.bf16_dev(q_bits), G.dev(np.asarray(pos, np.int32)), G.dev(cs), G.dev(w), w_scale, qp, qs,
                        wo)
    torch.cuda.synchronize()
    return qp.cpu().numpy(), qs.cpu().numpy(), wo.cpu().numpy()


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_q_prep_workloads_bit_exact(cfg):
    """The workloads' query rows, each query token rotated at its position (the step's
    newest n_q tokens of each sequence), with the fold of head_dim^-1/2 * H^-1/2."""
    W = wl.make_workload(cfg)
    G.say(f"q prep cfg={cfg} tokens={W.rows} H={W.H}")
    q = W.q_rows.reshape(W.rows, W.H, 128)
    pos = np.array([max(W.valid_len(r) - 1, 0) for r in range(W.rows)], np.int32)
    w = W.w.reshape(W.rows, W.H)
    scale = float(np.float32(128 ** -0.5 * W.H ** -0.5))
    got = run(q, pos, W.cos_sin, w, scale)
    ref = oracle.q_prep_mxfp4(q, pos, W.cos_sin, w, scale)
    for g, r, name in zip(got, ref, ("packed", "scales", "weights")):
        assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), f"cfg{cfg}: {name} differ"


def test_q_prep_edges():
    """Heads not a multiple of 16, positions outside the table (unrotated), extreme
    magnitudes (bf16 near its range and subnormal-scale blocks), zero vectors, a zero
    weight factor, and an empty call."""
    rng = np.random.default_rng(77)
    T, H = 7, 20
    x = rng.standard_normal((T, H, 128)).astype(np.float32)
    x[0, 0] *= 1e30
    x[0, 1] *= 1e-30
    x[1, 2] = 0.0
    x[2, 3, ::2] = -0.0
    q = wl.f32_to_bf16_bits(x)
    cs = wl.rope_cos_sin(64)
    pos = np.array([0, 63, 64, -1, 5, 1 << 30, 17], np.int32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    for scale in (0.0883883461356163, 0.0, 1.0):
        got = run(q, pos, cs, w, scale)
        ref = oracle.q_prep_mxfp4(q, pos, cs, w, scale)
        for g, r, name in zip(got, ref, ("packed", "scales", "weights")):
            assert np.array_equal(g.view(np.uint8), r.view(np.uint8)), f"scale {scale}: {name} differ"
    torch = G.torch_cuda()
    e = torch.empty((0,), device="cuda")
    bd.idx_q_prep_mxfp4(torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda"), e.int(), G.dev(cs),
                        e.reshape(0, H), 1.0, e.byte(), e.byte(), e)
    torch.cuda.synchronize()
