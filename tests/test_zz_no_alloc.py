"""GPU tier: vit_encode_varlen_noalloc (its workspace is the library's fixed
per-GPU array, so the call allocates nothing) against vit_encode_varlen with a
caller workspace, through the C ABI.  Same kernels and arithmetic, so the outputs
must be bitwise equal; two calls in a row, the second with a smaller input (the
array then still holds the first call's contents)."""
import ctypes

import pytest
import torch

from vision_transformer_encoder_image_amd import _lib, api, configs, synth

pytestmark = pytest.mark.gpu


def _inputs(name, n_images=None):
    cfg = configs.get(name)
    idx = [c.name for c in configs.CONFIGS].index(cfg.name)
    inp = synth.make_inputs(cfg, seed=idx)
    grids = list(cfg.grids) if n_images is None else list(cfg.grids)[:n_images]
    P = sum(h * w for h, w in grids)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"][:P]).to("cuda", torch.bfloat16)
    return cfg, w, x, grids


def _noalloc(cfg, w, x, grids, out):
    lib = _lib.load()
    flags = 0 if cfg.aligner else _lib.VIT_NO_ALIGNER
    c = api.c_config(cfg)
    return lib.vit_encode_varlen_noalloc(ctypes.byref(c), ctypes.byref(w.c), x.data_ptr(),
                                         _lib.grid_array(grids), len(grids), flags,
                                         out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def _check_equal(cfg, w, x, grids, tag):
    ref = api.Encoder(cfg, w, grids, aligner=cfg.aligner)(x)
    got = torch.full_like(ref, float("nan"))
    print(f"{tag}: {cfg.name} grids={grids}", flush=True)
    assert _noalloc(cfg, w, x, grids, got) == _lib.VIT_OK, _lib.load().vit_last_error()
    torch.cuda.synchronize()
    assert torch.equal(got, ref), f"{tag}: max abs diff {(got.float() - ref.float()).abs().max()}"


def test_noalloc_two_calls_match_workspace_entry_point():
    lib = _lib.load()
    assert lib.vit_noalloc_workspace_limit() == 160 << 20
    # the ragged 4-image batch, then a smaller input (two of its images)
    cfg, w, x, grids = _inputs("ragged_varlen_4img")
    _check_equal(cfg, w, x, grids, "first call")
    cfg, w, x, grids = _inputs("ragged_varlen_4img", n_images=2)
    _check_equal(cfg, w, x, grids, "second call")


def test_noalloc_near_limit_and_with_aligner():
    """The 64x64 full tower with its aligner needs ~129 MB of the 160 MiB."""
    cfg, w, x, grids = _inputs("highres_64x64_full_tower")
    assert api.workspace_bytes(cfg, grids, aligner=True) <= 160 << 20
    _check_equal(cfg, w, x, grids, "near the limit")
    cfg, w, x, grids = _inputs("single_28x28")
    _check_equal(cfg, w, x, grids, "smaller, after it")


def test_noalloc_rejects_oversize_without_enqueueing():
    """16 x 48x48 needs ~0.95 GB: rejected with VIT_E_WORKSPACE, output untouched."""
    cfg, w, x, grids = _inputs("throughput_16x48x48")
    lib = _lib.load()
    assert api.workspace_bytes(cfg, grids, aligner=True) > lib.vit_noalloc_workspace_limit()
    out = torch.full((8, 8), 7.0, dtype=torch.bfloat16, device="cuda")
    st = _noalloc(cfg, w, x, grids, out)
    torch.cuda.synchronize()
    assert st == _lib.VIT_E_WORKSPACE
    assert b"167772160" in lib.vit_last_error()
    assert torch.equal(out, torch.full_like(out, 7.0))
