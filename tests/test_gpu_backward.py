"""GPU tier: vit_mlp_backward (gradients of the MLP half of a block) against
oracle.mlp_half_backward on seeded inputs, float64 reference."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, rowwise_rel_err, to_np
from vision_transformer_encoder_image_amd import _lib, api, synth

pytestmark = pytest.mark.gpu


def _case(P, d, h, seed):
    x = synth.random_array((P, d), seed, std=1.0)
    w = np.float32(1.0) + synth.random_array((d,), seed + 1, std=0.02)
    wg = synth.random_array((h, d), seed + 2, std=0.02, bf16=True)
    wu = synth.random_array((h, d), seed + 3, std=0.02, bf16=True)
    wd = synth.random_array((d, h), seed + 4, std=0.02, bf16=True)
    dy = synth.random_array((P, d), seed + 5, std=1.0)
    return x, w, wg, wu, wd, dy


def _run(x, w, wg, wu, wd, dy, eps=1e-6):
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    b = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16)
    out = api.mlp_backward(f(x), f(w), b(wg), b(wu), b(wd), f(dy), eps)
    torch.cuda.synchronize()
    return [to_np(t) for t in out]


def _check(got, ref, tag, whole_matrix_weights=False):
    """Row-wise relative error (the encoder's bar).  With a single row every weight
    gradient row is one product scaled by one entry of da = dy W_down, whose bf16
    operand rounding leaves a cancelling entry with a large relative error; that
    case measures the weight gradients against the whole matrix instead."""
    names = ["dx", "d_norm_w", "d_w_gate", "d_w_up", "d_w_down"]
    for name, g, r in zip(names, got, ref):
        assert g.shape == r.shape, name
        g2, r2 = (g[None], r[None]) if g.ndim == 1 else (g, r)
        if whole_matrix_weights and name.startswith("d_w_"):
            g2, r2 = g2.reshape(1, -1), r2.reshape(1, -1)
        err = rowwise_rel_err(g2, r2)
        print(f"{tag} {name}: row-wise rel err {err:.3e}")
        assert err < TOL["bf16"], (name, err)


@pytest.mark.parametrize("P,d,h", [(300, 256, 512), (64, 128, 192), (1, 64, 64)])
def test_mlp_backward_small_matches_oracle(P, d, h):
    args = _case(P, d, h, seed=70 + P)
    _check(_run(*args), oracle.mlp_half_backward(*args), f"P={P} d={d} h={h}",
           whole_matrix_weights=P == 1)


def test_mlp_backward_ragged_batch_shape_matches_oracle():
    """The ragged 4-image batch's rows and widths: 3562 x 1024, hidden 2816."""
    args = _case(3562, 1024, 2816, seed=80)
    _check(_run(*args), oracle.mlp_half_backward(*args), "3562x1024x2816")


def test_mlp_backward_deterministic():
    args = _case(777, 256, 320, seed=90)
    a, b = _run(*args), _run(*args)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_mlp_backward_error_paths():
    lib = _lib.load()
    assert lib.vit_mlp_backward_workspace_bytes(100, 96, 128) == 0  # dim % 64
    assert lib.vit_mlp_backward_workspace_bytes(100, 128, 100) == 0  # hidden % 64
    assert lib.vit_mlp_backward_workspace_bytes(0, 128, 128) == 0
    assert lib.vit_mlp_backward(None, None, 0, None) == _lib.VIT_E_ARG
    t = torch.zeros(64 * 64, device="cuda")
    a = _lib.VitMlpGrad(16, 64, 64, 1e-6, *([t.data_ptr()] * 11))
    assert lib.vit_mlp_backward(a, t.data_ptr(), 16, torch.cuda.current_stream().cuda_stream) == \
        _lib.VIT_E_WORKSPACE


# ---------------------------------------------------------------- attention half
def _attn_case(grids, d, seed):
    P = sum(h * w for h, w in grids)
    x = synth.random_array((P, d), seed, std=1.0)
    w = np.float32(1.0) + synth.random_array((d,), seed + 1, std=0.02)
    wqkv = synth.random_array((3 * d, d), seed + 2, std=0.05, bf16=True)
    wo = synth.random_array((d, d), seed + 3, std=0.02, bf16=True)
    dy = synth.random_array((P, d), seed + 4, std=1.0)
    return x, w, wqkv, wo, dy


def _attn_oracle(x, w, wqkv, wo, dy, grids, H, theta=10000.0, eps=1e-6):
    dxs, dw, dwqkv, dwo, off = [], 0.0, 0.0, 0.0, 0
    for gh, gw in grids:
        P = gh * gw
        cos, sin = oracle.rope_table(gh, gw, x.shape[1] // H, theta)
        r = oracle.attn_half_backward(x[off:off + P], w, wqkv, wo, cos, sin, H, dy[off:off + P], eps)
        dxs.append(r[0])
        dw, dwqkv, dwo = dw + r[1], dwqkv + r[2], dwo + r[3]
        off += P
    return [np.concatenate(dxs), dw, dwqkv, dwo]


def _attn_run(x, w, wqkv, wo, dy, grids, H):
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    b = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16)
    out = api.attn_backward(f(x), f(w), b(wqkv), b(wo), f(dy), grids, H)
    torch.cuda.synchronize()
    return [to_np(t) for t in out]


# Bar of the attention half's gradients, from the arithmetic: about six bf16
# roundings of operands chained through the gradient (n, q k v, dO, P and dS, the
# outputs; 2^-9 each, ~1.2e-2 if they add up) and the cancellation in
# dS = P (dP - rowsum(dO o)), with o the bf16 attention output as saved by the
# forward: 3e-2.  Measured 1e-2 .. 2e-2 on these cases.
ATTN_GRAD_TOL = 3e-2


def _attn_check(got, ref, tag, whole_matrix_weights=False):
    """Row-wise relative error; with very few rows (whole_matrix_weights) each
    weight-gradient row is a sum of a handful of products that can nearly cancel,
    so the weight gradients are measured against the whole matrix instead."""
    for name, g, r in zip(["dx", "d_norm_w", "d_wqkv", "d_wo"], got, ref):
        assert g.shape == r.shape, name
        g2, r2 = (g[None], r[None]) if g.ndim == 1 else (g, r)
        if whole_matrix_weights and name in ("d_wqkv", "d_wo"):
            g2, r2 = g2.reshape(1, -1), r2.reshape(1, -1)
        err = rowwise_rel_err(g2, r2)
        print(f"{tag} {name}: row-wise rel err {err:.3e}")
        assert err < ATTN_GRAD_TOL, (name, err)


@pytest.mark.parametrize("grids", [[(4, 6), (3, 5), (8, 8)], [(1, 1), (2, 3)], [(4, 17)]])
def test_attn_backward_small_grids_match_oracle(grids):
    H, d = 2, 128
    args = _attn_case(grids, d, seed=110 + len(grids))
    rows = sum(h * w for h, w in grids)
    _attn_check(_attn_run(*args, grids, H), _attn_oracle(*args, grids, H), f"{grids}",
                whole_matrix_weights=rows < 64)


def test_attn_backward_ragged_batch_matches_oracle():
    """The ragged 4-image batch: 27x37, 37x27, 10x78, 112x7, 16 heads x 64."""
    grids = [(27, 37), (37, 27), (10, 78), (112, 7)]
    H, d = 16, 1024
    args = _attn_case(grids, d, seed=120)
    _attn_check(_attn_run(*args, grids, H), _attn_oracle(*args, grids, H), "ragged batch")


def test_attn_backward_deterministic_and_errors():
    grids = [(6, 10), (5, 5)]
    args = _attn_case(grids, 128, seed=130)
    a, b = _attn_run(*args, grids, 2), _attn_run(*args, grids, 2)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    lib = _lib.load()
    bad = _lib.VitAttnGrad(96, 2, 1e4, 1e-6, *([None] * 9))  # head_dim 48
    assert lib.vit_attn_backward_workspace_bytes(bad, _lib.grid_array(grids), 2) == 0
    assert lib.vit_attn_backward(bad, _lib.grid_array(grids), 2, None, 0, None) == _lib.VIT_E_SHAPE
