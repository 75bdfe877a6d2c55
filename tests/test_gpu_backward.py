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
