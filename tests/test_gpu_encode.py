"""GPU tier, whole path: vit_encode / vit_encode_varlen against the oracle on the
five seeded workloads, plus determinism, newline-layout output and error paths."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, global_rel_err, rowwise_rel_err, to_np
from vision_transformer_encoder_image_amd import _lib, api, configs, synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_cache = {}


def _setup(idx):
    if idx not in _cache:
        cfg = configs.get(idx)
        inp = synth.make_inputs(cfg, seed=idx)
        w = api.DeviceWeights(cfg, inp["weights"])
        x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16 if cfg.dtype == "bf16"
                                                  else torch.float32)
        _cache.clear()
        _cache[idx] = (cfg, inp, w, x)
    return _cache[idx]


def _oracle(cfg, inp, grids=None, patches=None):
    return oracle.encode_varlen(inp["patches"] if patches is None else patches,
                                inp["grids"] if grids is None else grids, inp["weights"],
                                cfg.n_heads, cfg.rms_eps, cfg.rope_theta, with_aligner=cfg.aligner)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_workload_full_parity(idx):
    cfg, inp, w, x = _setup(idx)
    got = to_np(api.Encoder(cfg, w, cfg.grids, aligner=cfg.aligner)(x))
    ref = _oracle(cfg, inp)
    assert got.shape == ref.shape
    err = rowwise_rel_err(got, ref)
    print(f"{cfg.name}: row-wise rel err {err:.3e}, global {global_rel_err(got, ref):.3e}")
    assert err < TOL[cfg.dtype], err


def test_highres_full_tower_against_stored_oracle():
    """64x64 grid, 32 blocks, head_dim 72: every aligner output row against the stored
    oracle run (tests/golden/make_expected.py), whose inputs must be the ones the
    seeded generator gives today."""
    import sys

    sys.path.insert(0, GOLDEN)
    import make_expected

    path = os.path.join(GOLDEN, "expected_highres_64x64_full_tower.npz")
    ref = np.load(path)
    cfg, inp, w, x = _setup(3)
    assert str(ref["fingerprint"]) == make_expected.fingerprint(inp), "stored oracle inputs drifted"
    got = to_np(api.Encoder(cfg, w, cfg.grids, aligner=True)(x))
    assert tuple(ref["shape"]) == got.shape
    rows = ref["rows"]
    assert len(rows) == got.shape[0], "the stored run covers every output row"
    per_row = np.abs(got[rows] - ref["values"]).max(1) / np.abs(ref["values"]).max(1)
    err = float(per_row.max())
    print(f"{cfg.name}: row-wise rel err max {err:.3e} (row {int(rows[per_row.argmax()])}), "
          f"median {float(np.median(per_row)):.3e}, margin to the bar {TOL['bf16'] - err:.3e}, "
          f"{len(rows)} rows")
    assert err < TOL["bf16"], err


@pytest.fixture(scope="module")
def throughput_out():
    cfg, inp, w, x = _setup(4)
    return to_np(api.Encoder(cfg, w, cfg.grids, aligner=True)(x)), inp


@pytest.mark.parametrize("image", range(16))
def test_throughput_batch_every_image(throughput_out, image):
    """16 x 48x48 images: images are independent, so the oracle runs one image at a
    time, each against its rows of the whole-batch call; together the 16 cases cover
    every output row."""
    cfg = configs.get(4)
    got, inp = throughput_out
    P, T = 48 * 48, 24 * 24
    i = image
    ref = _oracle(cfg, inp, grids=[(48, 48)], patches=inp["patches"][i * P:(i + 1) * P])
    err = rowwise_rel_err(got[i * T:(i + 1) * T], ref)
    print(f"{cfg.name} image {i}: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err


def test_single_image_entry_matches_varlen_bitwise():
    cfg, inp, w, x = _setup(1)
    a = api.encode(x, cfg.grids[0], w, aligner=True)
    b = api.encode_varlen(x, cfg.grids, w, aligner=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _unpatchify(patches, grids, ps=14):
    """Pixel images [3, ps*gh, ps*gw] (flattened, back to back) whose patches are
    the given rows; pinned against oracle.patchify below."""
    out, off = [], 0
    for gh, gw in grids:
        P = gh * gw
        img = (patches[off:off + P].reshape(gh, gw, 3, ps, ps).transpose(2, 0, 3, 1, 4)
               .reshape(3, gh * ps, gw * ps))
        np.testing.assert_array_equal(oracle.patchify(img, ps), patches[off:off + P])
        out.append(img.reshape(-1))
        off += P
    return np.concatenate(out)


@pytest.mark.parametrize("idx", [0, 2])
def test_pixel_input_matches_patch_input(idx):
    """VIT_IN_PIXELS: the library cuts the pixel images into the patches the
    oracle's patchify gives, so the result equals the patch-input call bitwise."""
    cfg, inp, w, x = _setup(idx)
    pix = _unpatchify(np.asarray(inp["patches"]), cfg.grids)
    xp = torch.from_numpy(pix).to("cuda", x.dtype)
    a = api.Encoder(cfg, w, cfg.grids, aligner=cfg.aligner)(x)
    b = api.Encoder(cfg, w, cfg.grids, aligner=cfg.aligner, pixels=True)(xp)
    c = api.encode(xp, cfg.grids[0], w, aligner=cfg.aligner, pixels=True) if len(cfg.grids) == 1 \
        else None
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    if c is not None:
        assert torch.equal(a, c)


def test_deterministic_run_to_run():
    cfg, inp, w, x = _setup(2)
    enc = api.Encoder(cfg, w, cfg.grids, aligner=False)
    a = enc(x).clone()
    b = enc(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_varlen_equals_per_image_runs():
    cfg, inp, w, x = _setup(2)
    whole = to_np(api.Encoder(cfg, w, cfg.grids, aligner=False)(x))
    off = 0
    for gh, gw in cfg.grids:
        P = gh * gw
        one = to_np(api.encode(x[off:off + P].contiguous(), (gh, gw), w, aligner=False))
        np.testing.assert_array_equal(one, whole[off:off + P])
        off += P


def test_newline_layout_output():
    cfg, inp, w, x = _setup(1)
    plain = api.encode(x, cfg.grids[0], w, aligner=True)
    nl = api.encode(x, cfg.grids[0], w, aligner=True, nlayout=True)
    torch.cuda.synchronize()
    types, src = oracle.nlayout(*cfg.grids[0])
    img = types == 1
    assert nl.shape[0] == len(types)
    assert torch.equal(nl[torch.from_numpy(np.nonzero(img)[0]).cuda()], plain[torch.from_numpy(src[img]).long().cuda()])
    assert (nl[torch.from_numpy(np.nonzero(~img)[0]).cuda()] == 0).all()  # sentinel rows untouched


def test_tiny_and_ragged_edge_grids():
    """1x1, 1xN and tall grids in one bf16 batch (encoder only), against the oracle."""
    cfg = configs.VitConfig("edge", ((1, 1), (1, 17), (33, 2), (5, 5)), 256, 4, 704, 2, 0, "bf16")
    inp = synth.make_inputs(cfg, seed=99)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.Encoder(cfg, w, cfg.grids, aligner=False)(x))
    ref = _oracle(cfg, inp)
    assert rowwise_rel_err(got, ref) < TOL["bf16"]


def test_max_images_per_call():
    cfg = configs.VitConfig("many", tuple([(2, 2)] * _lib.VIT_MAX_IMAGES), 256, 4, 704, 1, 512, "bf16")
    inp = synth.make_inputs(cfg, seed=98)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.Encoder(cfg, w, cfg.grids, aligner=True)(x))
    for i in (0, 77, _lib.VIT_MAX_IMAGES - 1):
        ref = _oracle(cfg, inp, grids=[(2, 2)], patches=inp["patches"][4 * i:4 * i + 4])
        assert rowwise_rel_err(got[i:i + 1], ref) < TOL["bf16"]


def test_error_paths_on_device():
    cfg, inp, w, x = _setup(1)
    enc = api.Encoder(cfg, w, cfg.grids, aligner=True)
    lib = _lib.load()
    out = torch.empty(enc.out_shape, dtype=torch.bfloat16, device="cuda")
    st = lib.vit_encode(ctypes.byref(enc.c_cfg), ctypes.byref(w.c), x.data_ptr(), 27, 37, 0,
                        out.data_ptr(), enc.ws.data_ptr(), enc.ws_bytes,
                        torch.cuda.current_stream().cuda_stream)
    assert st == _lib.VIT_E_ODD_GRID
    out = torch.empty(enc.out_shape, dtype=torch.bfloat16, device="cuda")
    st = lib.vit_encode_varlen(ctypes.byref(enc.c_cfg), ctypes.byref(w.c), x.data_ptr(), enc.c_grids,
                               1, enc.flags, out.data_ptr(), enc.ws.data_ptr(), enc.ws_bytes - 256,
                               torch.cuda.current_stream().cuda_stream)
    assert st == _lib.VIT_E_WORKSPACE


def _ragged_aligned_cfg():
    # the ragged 4-image grids (three of them odd) with a 512-wide aligner, 2 blocks
    return configs.VitConfig("ragged_aligned", ((27, 37), (37, 27), (10, 78), (112, 7)),
                             1024, 16, 2816, 2, 512, "bf16")


def test_odd_grids_zero_padded_aligner_matches_oracle():
    cfg = _ragged_aligned_cfg()
    inp = synth.make_inputs(cfg, seed=97)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.Encoder(cfg, w, cfg.grids, aligner=True, pad_odd=True)(x))
    ref = oracle.encode_varlen(inp["patches"], inp["grids"], inp["weights"], cfg.n_heads,
                               cfg.rms_eps, cfg.rope_theta, with_aligner=True, pad_odd=True)
    assert got.shape == ref.shape == (14 * 19 + 19 * 14 + 5 * 39 + 56 * 4, 512)
    err = rowwise_rel_err(got, ref)
    print(f"odd grids, zero-padded aligner: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err
    # without the flag the odd grids are still refused
    with pytest.raises(_lib.VitError):
        api.Encoder(cfg, w, cfg.grids, aligner=True)


def test_odd_grids_newline_layout_rows():
    cfg = _ragged_aligned_cfg()
    inp = synth.make_inputs(cfg, seed=97)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    plain = api.Encoder(cfg, w, cfg.grids, aligner=True, pad_odd=True)(x)
    nl = api.Encoder(cfg, w, cfg.grids, aligner=True, nlayout=True, pad_odd=True)(x)
    torch.cuda.synchronize()
    rows, toks = [], []
    base = tok = 0
    for gh, gw in cfg.grids:
        types, src = oracle.nlayout(gh, gw, pad_odd=True)
        img = np.nonzero(types == oracle.NL_IMAGE)[0]
        rows.append(base + img)
        toks.append(tok + src[img])
        base += len(types)
        tok += int((types == oracle.NL_IMAGE).sum())
    rows, toks = np.concatenate(rows), np.concatenate(toks)
    assert nl.shape[0] == base and plain.shape[0] == tok
    assert torch.equal(nl[torch.from_numpy(rows).long().cuda()],
                       plain[torch.from_numpy(toks).long().cuda()])
    sentinel = np.setdiff1d(np.arange(base), rows)
    assert (nl[torch.from_numpy(sentinel).long().cuda()] == 0).all()


@pytest.mark.parametrize("idx", [1, 2])
def test_encode_replays_from_a_captured_graph(idx):
    """The encode call enqueues kernels only (no memset, copy or allocation), so a
    caller can capture it in a HIP graph: three replays, with eager encodes of
    other inputs through the same workspace and synchronizations between them,
    each equal bitwise to the eager result (28x28 with the aligner; the ragged
    batch without)."""
    cfg, inp, w, x = _setup(idx)
    enc = api.Encoder(cfg, w, cfg.grids, aligner=cfg.aligner)
    out = torch.empty(enc.out_shape, dtype=x.dtype, device="cuda")
    ref = enc(x).clone()
    enc(x, out)  # warm-up outside the capture (first-call kernel attributes)
    torch.cuda.synchronize()
    x_in = x.clone()
    other = torch.flip(x, [0]).contiguous()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc(x_in, out)
    for _ in range(3):
        out.zero_()
        junk = enc(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert not torch.equal(junk, ref)


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_ragged_batches_match_oracle(seed):
    """Randomised batches: 1-6 images of grids 1..24 x 1..24 (odd grids zero-padded
    for the 2x2 merge), width 128 (2 heads of 64), hidden 192, 2 blocks, 4x4
    patches, the aligner on or off; the whole path against the oracle at the
    workload bar."""
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    n = int(rng.integers(1, 7))
    grids = tuple((int(rng.integers(1, 25)), int(rng.integers(1, 25))) for _ in range(n))
    aligner = bool(seed % 2 == 0)
    cfg = configs.VitConfig(f"random{seed}", grids, 128, 2, 192, 2, 256 if aligner else 0, "bf16",
                            patch_size=4)
    inp = synth.make_inputs(cfg, seed=2000 + seed)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.encode_varlen(x, list(grids), w, aligner=aligner, pad_odd=aligner))
    ref = oracle.encode_varlen(inp["patches"], list(grids), inp["weights"], cfg.n_heads,
                               cfg.rms_eps, cfg.rope_theta, with_aligner=aligner, pad_odd=aligner)
    assert got.shape == ref.shape
    err = rowwise_rel_err(got, ref)
    print(f"seed {seed} grids {grids} aligner {aligner}: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err


@pytest.mark.parametrize("seed", list(range(4)))
def test_random_ragged_batches_head_dim_72(seed):
    """Randomised batches through the head_dim-72 path (width 576 = 8 heads of 72,
    the rotary applied by the V^T pack launch, the 16x16x32 attention kernel):
    1-6 images of grids 1..24 x 1..24, hidden 192, 2 blocks, 4x4 patches, the
    aligner on or off; the whole path against the oracle at the workload bar."""
    rng = np.random.Generator(np.random.PCG64(3000 + seed))
    n = int(rng.integers(1, 7))
    grids = tuple((int(rng.integers(1, 25)), int(rng.integers(1, 25))) for _ in range(n))
    aligner = bool(seed % 2 == 0)
    cfg = configs.VitConfig(f"random72_{seed}", grids, 576, 8, 192, 2, 256 if aligner else 0,
                            "bf16", patch_size=4)
    assert cfg.head_dim == 72
    inp = synth.make_inputs(cfg, seed=4000 + seed)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.encode_varlen(x, list(grids), w, aligner=aligner, pad_odd=aligner))
    ref = oracle.encode_varlen(inp["patches"], list(grids), inp["weights"], cfg.n_heads,
                               cfg.rms_eps, cfg.rope_theta, with_aligner=aligner, pad_odd=aligner)
    assert got.shape == ref.shape
    err = rowwise_rel_err(got, ref)
    print(f"seed {seed} grids {grids} aligner {aligner}: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err


@pytest.mark.parametrize("width,heads", [(128, 2), (576, 8)], ids=["head_dim64", "head_dim72"])
def test_large_image_long_sequence(width, heads):
    """One 96x96 image (9,216 patches: 145 key tiles per query, rotary positions up
    to 95) beside a 3x5 image, one block, the aligner on (the odd grid zero-padded),
    through the head_dim-64 and head_dim-72 paths; the whole output against the
    oracle at the workload bar."""
    grids = ((96, 96), (3, 5))
    cfg = configs.VitConfig(f"large_{width}", grids, width, heads, 192, 1, 256, "bf16", patch_size=4)
    assert cfg.head_dim in (64, 72)
    inp = synth.make_inputs(cfg, seed=77)
    w = api.DeviceWeights(cfg, inp["weights"])
    x = torch.from_numpy(inp["patches"]).to("cuda", torch.bfloat16)
    got = to_np(api.encode_varlen(x, list(grids), w, aligner=True, pad_odd=True))
    ref = oracle.encode_varlen(inp["patches"], list(grids), inp["weights"], cfg.n_heads,
                               cfg.rms_eps, cfg.rope_theta, with_aligner=True, pad_odd=True)
    assert got.shape == ref.shape
    err = rowwise_rel_err(got, ref)
    print(f"{cfg.name}: row-wise rel err {err:.3e}")
    assert err < TOL["bf16"], err
