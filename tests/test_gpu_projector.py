"""GPU tier: the PatchMerger projector (vit_patch_merger and its steps
vit_layernorm_gather / vit_gemm_bias) against the oracle on seeded inputs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, rowwise_rel_err, to_np
from vision_transformer_encoder_image_amd import _lib, api, synth

pytestmark = pytest.mark.gpu

# one bf16 output rounding per element (2^-9 relative) plus fp32 accumulation
STEP_TOL = 8e-3


def _dev(a, bf16=True):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        "cuda", torch.bfloat16 if bf16 else torch.float32)


def _oracle_varlen(x, grids, p, eps=1e-6):
    outs, off = [], 0
    for gh, gw in grids:
        P = gh * gw
        outs.append(oracle.patch_merger(x[off:off + P], gh, gw, p, eps))
        off += P
    return np.concatenate(outs)


@pytest.mark.parametrize("dim", [256, 1152])
def test_layernorm_gather_matches_oracle(dim):
    grids = [(4, 6), (2, 2), (8, 10), (6, 2)]
    P = sum(h * w for h, w in grids)
    x = synth.random_array((P, dim), 40 + dim, std=1.5, bf16=True) + np.float32(0.25)
    x = synth.round_to_bf16(x)
    w = synth.make_merger_weights(dim, 64, 8, seed=41)
    G = to_np(api.layernorm_gather(_dev(x), grids, _dev(w["ln_w"], False), _dev(w["ln_b"], False)))
    ref, off = [], 0
    for gh, gw in grids:
        n = oracle.layernorm(x[off:off + gh * gw], w["ln_w"], w["ln_b"], 1e-6)
        ref.append(oracle.aligner_gather(n, gh, gw))
        off += gh * gw
    ref = np.concatenate(ref)
    assert G.shape == ref.shape
    err = rowwise_rel_err(G, ref)
    print(f"layernorm+gather dim {dim}: row-wise rel err {err:.3e}")
    assert err < STEP_TOL, err


@pytest.mark.parametrize("gelu", [False, True])
# (3000, 5632, 256) takes a column split: 256x256 tiles over 5376 columns, the
# rest (bias offset by the split) in a second launch of 128x128 tiles
@pytest.mark.parametrize("shape", [(130, 200, 128), (257, 4096, 256), (64, 4608, 4608),
                                   (3000, 5632, 256)])
def test_gemm_bias_matches_oracle(shape, gelu):
    M, N, K = shape
    A = synth.random_array((M, K), 42, bf16=True)
    B = synth.random_array((N, K), 43, std=0.03, bf16=True)
    bias = synth.random_array((N,), 44, std=0.5)
    got = to_np(api.gemm_bias(_dev(A), _dev(B), _dev(bias, False), gelu=gelu))
    ref = oracle.linear(A, B) + bias
    if gelu:
        ref = oracle.gelu(ref)
    err = rowwise_rel_err(got, ref)
    print(f"gemm bias {shape} gelu={gelu}: row-wise rel err {err:.3e}")
    assert err < STEP_TOL, err


def test_patch_merger_small_matches_oracle():
    grids = [(4, 6), (2, 8), (6, 6)]
    dim, hidden, out = 256, 512, 384
    P = sum(h * w for h, w in grids)
    x = synth.random_array((P, dim), 45, bf16=True)
    w = synth.make_merger_weights(dim, hidden, out, seed=46)
    mw = api.MergerWeights(w)
    got = to_np(api.patch_merger(_dev(x), grids, mw))
    ref = _oracle_varlen(x, grids, w)
    assert got.shape == ref.shape == (P // 4, out)
    err = rowwise_rel_err(got, ref)
    print(f"patch merger small: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err


def test_patch_merger_page_shape_sampled_tokens():
    """1152-dim patches of a 64x64 grid -> 4608 -> 4096 (the page's projector on the
    high-res workload's tower width).  Merged tokens depend only on their own 2x2
    group, so the oracle runs on the top two and bottom two patch rows."""
    gh = gw = 64
    dim, hidden, out = 1152, 4608, 4096
    x = synth.random_array((gh * gw, dim), 47, bf16=True)
    w = synth.make_merger_weights(dim, hidden, out, seed=48)
    mw = api.MergerWeights(w)
    got = to_np(api.patch_merger(_dev(x), [(gh, gw)], mw))
    assert got.shape == (gh * gw // 4, out)
    top = oracle.patch_merger(x[:2 * gw], 2, gw, w)
    bottom = oracle.patch_merger(x[(gh - 2) * gw:], 2, gw, w)
    err = max(rowwise_rel_err(got[:gw // 2], top), rowwise_rel_err(got[-gw // 2:], bottom))
    print(f"patch merger 64x64 / 1152 -> 4608 -> 4096: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err


def test_patch_merger_deterministic_and_workspace_reuse():
    grids = [(8, 8), (4, 2)]
    dim, hidden, out = 256, 256, 128
    P = sum(h * w for h, w in grids)
    x = _dev(synth.random_array((P, dim), 49, bf16=True))
    mw = api.MergerWeights(synth.make_merger_weights(dim, hidden, out, seed=50))
    lib = _lib.load()
    g = _lib.grid_array(grids)
    ws = torch.empty(lib.vit_patch_merger_workspace_bytes(ctypes.byref(mw.c), g, len(grids)),
                     dtype=torch.uint8, device="cuda")
    a = api.patch_merger(x, grids, mw, ws=ws).clone()
    b = api.patch_merger(x, grids, mw, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_patch_merger_error_paths():
    lib = _lib.load()
    mw = api.MergerWeights(synth.make_merger_weights(256, 256, 128, seed=51))
    odd = _lib.grid_array([(3, 4)])
    assert lib.vit_patch_merger_workspace_bytes(ctypes.byref(mw.c), odd, 1) == 0
    x = torch.zeros((12, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((3, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.vit_patch_merger(ctypes.byref(mw.c), x.data_ptr(), odd, 1, out.data_ptr(), None, 0,
                                s) == _lib.VIT_E_ODD_GRID
    ok = _lib.grid_array([(2, 6)])
    assert lib.vit_patch_merger(ctypes.byref(mw.c), x.data_ptr(), ok, 1, out.data_ptr(), None, 0,
                                s) == _lib.VIT_E_WORKSPACE
