"""CPU tier: the C ABI library loads, exports every symbol declared in the
header, and rejects bad arguments on the host before any GPU work."""
import ctypes
import os
import re

import pytest

from vision_transformer_encoder_image_amd import _lib, api, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vitenc.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vit_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvitenc.so is not built; run __graft_entry__.build() first")
    return _lib.load()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("vit_encode", "vit_encode_varlen", "vit_workspace_bytes", "vit_aligner_layout",
              "vit_status_str", "vit_rmsnorm", "vit_rope", "vit_attention_varlen", "vit_gemm"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"{n} declared in vitenc.h but not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def test_status_strings(lib):
    assert lib.vit_status_str(0) == b"ok"
    assert b"workspace" in lib.vit_status_str(-4)
    assert lib.vit_status_str(12345) == b"unknown status"


def test_config_struct_layout():
    assert ctypes.sizeof(_lib.VitConfig) == 44
    assert ctypes.sizeof(_lib.VitWeights) == 10 * ctypes.sizeof(ctypes.c_void_p)


def test_host_validation_errors(lib):
    cfg = api.c_config(configs.get(1))
    g = _lib.grid_array([(28, 28)])
    # null config / weights / buffers -> VIT_E_ARG, before any device work
    assert lib.vit_encode(None, None, None, 28, 28, 0, None, None, 0, None) == _lib.VIT_E_ARG
    assert lib.vit_encode(ctypes.byref(cfg), None, None, 28, 28, 0, None, None, 0, None) == _lib.VIT_E_ARG
    # odd grid with the aligner on
    assert lib.vit_aligner_layout(27, 37, 2, None, None, None, None) == _lib.VIT_E_ODD_GRID
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), _lib.grid_array([(27, 37)]), 1, 0) == 0
    assert b"not divisible" in lib.vit_last_error()
    # the same grid is fine without the aligner, or with the zero-padding rule
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), _lib.grid_array([(27, 37)]), 1,
                                   _lib.VIT_NO_ALIGNER) > 0
    padded = lib.vit_workspace_bytes(ctypes.byref(cfg), _lib.grid_array([(27, 37)]), 1,
                                     _lib.VIT_ALIGN_PAD)
    even = lib.vit_workspace_bytes(ctypes.byref(cfg), _lib.grid_array([(28, 38)]), 1, 0)
    assert padded > 0 and padded <= even  # 14 x 19 merged tokens either way, fewer patches
    # bad shapes
    bad = api.c_config(configs.get(1))
    bad.head_dim = 60
    assert lib.vit_workspace_bytes(ctypes.byref(bad), g, 1, 0) == 0
    bad = api.c_config(configs.get(1))
    bad.n_heads = 8  # 8 * 64 != 1024
    assert lib.vit_workspace_bytes(ctypes.byref(bad), g, 1, 0) == 0
    # image count limits
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), g, 0, 0) == 0
    many = _lib.grid_array([(2, 2)] * (_lib.VIT_MAX_IMAGES + 1))
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), many, _lib.VIT_MAX_IMAGES + 1, 0) == 0
    ok = _lib.grid_array([(2, 2)] * _lib.VIT_MAX_IMAGES)
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), ok, _lib.VIT_MAX_IMAGES, 0) > 0
    # pixel input: patch_dim must be 3 * ps^2; unknown flags are refused
    px = api.c_config(configs.get(1))
    assert lib.vit_workspace_bytes(ctypes.byref(px), g, 1, _lib.VIT_IN_PIXELS) > 0
    px.patch_dim = 592  # 3 * ps^2 has no integer ps
    assert lib.vit_workspace_bytes(ctypes.byref(px), g, 1, _lib.VIT_IN_PIXELS) == 0
    assert b"3*ps^2" in lib.vit_last_error()
    assert lib.vit_encode(ctypes.byref(px), None, None, 28, 28, _lib.VIT_IN_PIXELS, None, None, 0,
                          None) == _lib.VIT_E_SHAPE
    assert lib.vit_workspace_bytes(ctypes.byref(cfg), g, 1, 64) == 0
    # GEMM argument checks (host side)
    assert lib.vit_gemm(0, 0, None, 8, None, None, 8, None, 8, 1, 1, 8, None) == _lib.VIT_E_ARG
    assert lib.vit_gemm(0, 9, 16, 8, 16, None, 8, 16, 8, 1, 1, 8, None) == _lib.VIT_E_ARG
    assert lib.vit_gemm(0, 0, 16, 12, 16, None, 12, 16, 8, 1, 1, 12, None) == _lib.VIT_E_SHAPE
    assert lib.vit_gemm(0, 0, 8, 16, 16, None, 16, 16, 8, 1, 1, 16, None) == _lib.VIT_E_ARG  # misaligned


def test_merge_host_validation(lib):
    assert lib.vit_merge_workspace_bytes(-1) == 0
    assert lib.vit_merge_workspace_bytes(1 << 31) == 0
    assert lib.vit_merge_workspace_bytes(0) == 256  # never 0, which means an error
    # one int32 count per 256 positions, rounded up to 256 bytes
    assert lib.vit_merge_workspace_bytes(256 * 64) == 256
    assert lib.vit_merge_workspace_bytes(256 * 64 + 1) == 512
    m = lib.vit_merge_image_embeddings
    assert m(7, None, 10, 64, None, None, 0, None, None, None, 0, None) == _lib.VIT_E_ARG
    assert m(0, None, 10, 63, None, None, 0, None, None, None, 0, None) == _lib.VIT_E_SHAPE
    assert m(1, None, 10, 2, None, None, 0, None, None, None, 0, None) == _lib.VIT_E_SHAPE
    assert m(0, None, -1, 64, None, None, 0, None, None, None, 0, None) == _lib.VIT_E_SHAPE
    assert m(0, None, 10, 64, None, None, 0, None, None, None, 0, None) == _lib.VIT_E_ARG
    assert m(0, 256, 10, 64, 256, None, 3, 256, None, 256, 4096, None) == _lib.VIT_E_ARG
    assert m(0, 264, 10, 64, 256, 256, 3, 256, None, 256, 4096, None) == _lib.VIT_E_ARG


def test_projector_host_validation(lib):
    g = _lib.grid_array([(4, 6)])
    m = _lib.VitMerger(1152, 4608, 4096, 1e-6, None, None, None, None, None, None)
    T = 4 * 6 // 4
    want = (T * 4 * 1152 * 2 + 255) // 256 * 256 + (T * 4608 * 2 + 255) // 256 * 256
    assert lib.vit_patch_merger_workspace_bytes(ctypes.byref(m), g, 1) == want
    assert lib.vit_patch_merger_workspace_bytes(ctypes.byref(m), _lib.grid_array([(3, 6)]), 1) == 0
    assert b"not divisible" in lib.vit_last_error()
    for dim, hidden, out in ((1160, 4608, 4096), (1152, 4600, 4096), (1152, 4608, 4092), (0, 64, 8)):
        bad = _lib.VitMerger(dim, hidden, out, 1e-6, None, None, None, None, None, None)
        assert lib.vit_patch_merger_workspace_bytes(ctypes.byref(bad), g, 1) == 0
    assert lib.vit_patch_merger(None, None, g, 1, None, None, 0, None) == _lib.VIT_E_ARG
    assert lib.vit_patch_merger(ctypes.byref(m), None, g, 1, None, None, 0, None) == _lib.VIT_E_ARG
    assert lib.vit_layernorm_gather(None, g, 1, 1152, None, None, 1e-6, None, None) == _lib.VIT_E_ARG
    assert lib.vit_layernorm_gather(256, g, 1, 1156, 256, 256, 1e-6, 256, None) == _lib.VIT_E_SHAPE
    assert lib.vit_gemm_bias(0, 256, 64, 256, 64, 256, 256, 64, 8, 8, 64, None) == _lib.VIT_E_ARG
    assert lib.vit_gemm_bias(_lib.VIT_EPI_BIAS, 256, 64, 256, 64, None, 256, 64, 8, 8, 64,
                             None) == _lib.VIT_E_ARG
    # K must be a multiple of 64 for the MFMA path
    assert lib.vit_gemm_bias(_lib.VIT_EPI_BIAS, 256, 72, 256, 72, 256, 256, 64, 8, 8, 72,
                             None) == _lib.VIT_E_SHAPE


def test_pixel_input_workspace(lib):
    # fp32 pixel input needs a buffer for the cut patches; bf16 reuses the padded one
    tiny = configs.get(0)
    assert api.workspace_bytes(tiny, list(tiny.grids), pixels=True) > \
        api.workspace_bytes(tiny, list(tiny.grids))
    c = configs.get(2)
    assert api.workspace_bytes(c, list(c.grids), aligner=False, pixels=True) == \
        api.workspace_bytes(c, list(c.grids), aligner=False)


def test_workspace_grows_with_patches(lib):
    c = configs.get(2)
    small = api.workspace_bytes(c, [(8, 8)], aligner=False)
    big = api.workspace_bytes(c, list(c.grids), aligner=False)
    assert big > small > 0
    # the plan holds at least the fp32 residual stream and the qkv buffer
    P = c.total_patches
    assert big >= P * c.vision_dim * 4 + P * 3 * c.vision_dim * 2


def test_tower_backward_workspace_host_checks(lib):
    """Host-side sizing of vit_tower_backward: bf16 with head_dim 64 or 72, hidden a
    multiple of 16; the workspace holds at least the forward's plus 2 n_blocks + 1
    fp32 residual checkpoints."""
    c = configs.get(2)
    grids = list(c.grids)
    need = api.tower_backward_workspace_bytes(c, grids)
    P, d = c.total_patches, c.vision_dim
    assert need >= api.workspace_bytes(c, grids, aligner=False) + (2 * c.n_blocks + 1) * P * d * 4
    g = _lib.grid_array(grids)
    for bad in (configs.VitConfig("f", c.grids, 1024, 16, 2816, 4, 0, "f32"),
                configs.VitConfig("h", c.grids, 1024, 8, 2816, 4, 0, "bf16"),
                configs.VitConfig("m", c.grids, 1024, 16, 2808, 4, 0, "bf16")):
        assert lib.vit_tower_backward_workspace_bytes(ctypes.byref(api.c_config(bad)), g, 4) == 0
    # the 64x64 tower's widths (head_dim 72, hidden 4304) are taken
    c4 = configs.get(3)
    assert api.tower_backward_workspace_bytes(c4, list(c4.grids)) > 0
    one = api.tower_backward_workspace_bytes(
        configs.VitConfig("b1", c.grids, 1024, 16, 2816, 1, 0, "bf16"), grids)
    assert need - one >= 6 * P * d * 4


def test_mfma_probe_host_checks(lib):
    """vit_mfma_peak rejects NULL pointers and bad iteration counts on the host,
    before any launch; its output buffer size is a fixed, positive count."""
    flops = ctypes.c_double()
    assert lib.vit_mfma_peak(100, None, ctypes.byref(flops), None) == _lib.VIT_E_ARG
    assert lib.vit_mfma_peak(0, ctypes.c_void_p(16), ctypes.byref(flops), None) == _lib.VIT_E_ARG
    assert lib.vit_mfma_peak(1 << 25, ctypes.c_void_p(16), ctypes.byref(flops), None) == _lib.VIT_E_ARG
    assert lib.vit_mfma_peak_out_floats() == 256 * 512


def test_configs_flops_match_hand_count():
    c = configs.get(2)
    assert c.total_patches == 3562  # 999 + 999 + 780 + 784
    P, d, h = 3562, 1024, 2816
    attn = 4 * d * (999 ** 2 * 2 + 780 ** 2 + 784 ** 2)
    assert c.block_flops() == 8 * P * d * d + 6 * P * d * h + attn
