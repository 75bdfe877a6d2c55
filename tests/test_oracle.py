"""Pins of the CPU oracle against things other than itself.

Every function of ``oracle`` is checked here against closed forms, hand-worked
golden values under ``tests/golden/`` (each citing the page passage it follows),
brute-force scalar loops on tiny inputs, or invariants the method must satisfy
(norm preservation and (0,0)-identity of the rotary, shift invariance of the
attention logits, softmax rows summing to one, ...).  Each pin is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, swapped gate/up, a wrong merge order) fails at least one test.
"""
import math
import os

import numpy as np
import pytest

import oracle
from vision_transformer_encoder_image_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- linear / patchify
def test_linear_matches_scalar_loop():
    rng = _rng(1)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))  # [out, in]
    y = oracle.linear(x, w)
    assert y.shape == (3, 4)
    for i in range(3):
        for n in range(4):
            s = 0.0
            for k in range(5):
                s += x[i, k] * w[n, k]
            assert abs(y[i, n] - s) < 1e-12


def test_patchify_pixel_positions():
    gh, gw, ps = 2, 3, 14
    img = np.zeros((3, gh * ps, gw * ps), dtype=np.float64)
    for ch in range(3):
        for y in range(gh * ps):
            for x in range(gw * ps):
                img[ch, y, x] = ch * 100000 + y * 100 + x
    p = oracle.patchify(img, ps)
    assert p.shape == (gh * gw, 3 * ps * ps)
    for r in range(gh):
        for c in range(gw):
            for ch in range(3):
                for i in range(ps):
                    for j in range(ps):
                        e = ch * ps * ps + i * ps + j
                        assert p[r * gw + c, e] == ch * 100000 + (ps * r + i) * 100 + (ps * c + j)


# ---------------------------------------------------------------- RMSNorm
def _read_rms_golden():
    cases = []
    with open(os.path.join(GOLDEN, "rmsnorm_closed_form.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, rest = line.split(None, 1)
            xs, ws, ys = [np.array([float(t) for t in part.split()]) for part in rest.split("|")]
            cases.append((name, xs, ws, ys))
    return cases


@pytest.mark.parametrize("case", _read_rms_golden(), ids=lambda c: c[0])
def test_rmsnorm_golden(case):
    _, x, w, y = case
    got = oracle.rmsnorm(x[None], w, eps=1e-6)[0]
    np.testing.assert_allclose(got, y, rtol=1e-13, atol=1e-15)


def test_rmsnorm_unit_weight_mean_square():
    rng = _rng(2)
    x = rng.standard_normal((7, 33)) * 0.01
    y = oracle.rmsnorm(x, np.ones(33), eps=1e-6)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-6), rtol=1e-12)


def test_rmsnorm_scale_invariance():
    rng = _rng(3)
    x = rng.standard_normal((4, 64))
    w = 1 + 0.02 * rng.standard_normal(64)
    a = oracle.rmsnorm(x, w, eps=0.0)
    b = oracle.rmsnorm(37.5 * x, w, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12)


# ---------------------------------------------------------------- rotary
def test_rope_freqs_closed_form():
    f = oracle.rope_freqs(64, 10000.0)
    assert len(f) == 16
    assert f[0] == 1.0
    assert abs(f[8] - 0.01) < 1e-15  # 10000^(-8/16)
    assert abs(f[1] - 0.5623413251903491) < 1e-15  # 10000^(-1/16)
    f72 = oracle.rope_freqs(72, 10000.0)
    assert len(f72) == 18 and abs(f72[9] - 0.01) < 1e-15


def _read_rope_golden():
    rows = []
    with open(os.path.join(GOLDEN, "rope_unit_vectors.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            D, r, c, i, o, v = line.split()
            rows.append((int(D), int(r), int(c), int(i), int(o), float(v)))
    return rows


@pytest.mark.parametrize("row", _read_rope_golden())
def test_rope_unit_vectors_golden(row):
    D, r, c, i, o, v = row
    gw = c + 1
    gh = r + 1
    cos, sin = oracle.rope_table(gh, gw, D, 10000.0)
    p = r * gw + c
    x = np.zeros((1, 1, D))
    x[0, 0, i] = 1.0
    y = oracle.apply_rope(x, cos[p:p + 1], sin[p:p + 1])[0, 0]
    assert abs(y[o] - v) < 1e-14
    # exactly two non-zero outputs: the element itself and its rotate_half partner
    q = D // 4
    partner = i + q if (i % (D // 2)) < q else i - q
    for j in range(D):
        if j not in (i, partner):
            assert y[j] == 0.0


@pytest.mark.parametrize("D", [8, 64, 72])
def test_rope_identity_at_origin_and_norm_preserved(D):
    rng = _rng(4)
    gh, gw = 5, 7
    x = rng.standard_normal((gh * gw, 3, D))
    cos, sin = oracle.rope_table(gh, gw, D)
    y = oracle.apply_rope(x, cos, sin)
    np.testing.assert_array_equal(y[0], x[0])  # position (0, 0): identity
    q = D // 4
    for half in range(2):
        lo = half * D // 2
        n_in = x[..., lo:lo + q] ** 2 + x[..., lo + q:lo + 2 * q] ** 2
        n_out = y[..., lo:lo + q] ** 2 + y[..., lo + q:lo + 2 * q] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


def test_rope_half_separation():
    rng = _rng(5)
    D = 64
    x = rng.standard_normal((1, 2, D))
    # row only: second half untouched; column only: first half untouched
    cos, sin = oracle.rope_table(4, 1, D)  # patch 3 sits at (3, 0)
    y = oracle.apply_rope(x, cos[3:4], sin[3:4])
    np.testing.assert_array_equal(y[..., D // 2:], x[..., D // 2:])
    assert not np.allclose(y[..., :D // 2], x[..., :D // 2])
    cos, sin = oracle.rope_table(1, 4, D)  # patch 3 sits at (0, 3)
    y = oracle.apply_rope(x, cos[3:4], sin[3:4])
    np.testing.assert_array_equal(y[..., :D // 2], x[..., :D // 2])
    assert not np.allclose(y[..., D // 2:], x[..., D // 2:])


def test_rope_composition():
    rng = _rng(6)
    D = 72
    x = rng.standard_normal((1, 2, D))
    c1, s1 = oracle.rope_table(1, 1, D, origin=(3, 11))
    c2, s2 = oracle.rope_table(1, 1, D, origin=(40, -5))
    c3, s3 = oracle.rope_table(1, 1, D, origin=(43, 6))
    y12 = oracle.apply_rope(oracle.apply_rope(x, c1, s1), c2, s2)
    y3 = oracle.apply_rope(x, c3, s3)
    np.testing.assert_allclose(y12, y3, rtol=1e-11, atol=1e-12)


def test_rope_table_positions_restart_row_major():
    D = 8
    cos, sin = oracle.rope_table(3, 5, D)
    f = [1.0, 0.01]
    for p in range(15):
        r, c = divmod(p, 5)
        for k in range(2):
            assert abs(cos[p, k] - math.cos(r * f[k])) < 1e-15
            assert abs(sin[p, 2 + k] - math.sin(c * f[k])) < 1e-15


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v):
    P, H, D = q.shape
    out = np.zeros((P, H, D))
    for h in range(H):
        for i in range(P):
            logits = []
            for j in range(P):
                s = 0.0
                for e in range(D):
                    s += q[i, h, e] * k[j, h, e]
                logits.append(s / math.sqrt(D))
            m = max(logits)
            ws = [math.exp(t - m) for t in logits]
            tot = sum(ws)
            for j in range(P):
                for e in range(D):
                    out[i, h, e] += ws[j] / tot * v[j, h, e]
    return out


def test_attention_brute_force_4x4():
    rng = _rng(7)
    q, k, v = (rng.standard_normal((16, 2, 8)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v), _brute_attention(q, k, v),
                               rtol=1e-12, atol=1e-13)


def test_attention_rows_sum_to_one():
    rng = _rng(8)
    q, k = (rng.standard_normal((30, 3, 16)) * 3 for _ in range(2))
    a = oracle.attention_probs(q, k)
    np.testing.assert_allclose(a.sum(-1), 1.0, rtol=1e-13)
    assert (a > 0).all()


def test_attention_single_patch_and_equal_keys():
    rng = _rng(9)
    q, k, v = (rng.standard_normal((1, 2, 8)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v), v, rtol=1e-14)
    q = rng.standard_normal((6, 2, 8))
    k = np.repeat(rng.standard_normal((1, 2, 8)), 6, axis=0)
    v = rng.standard_normal((6, 2, 8))
    o = oracle.attention(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), rtol=1e-12)


def test_attention_permutation_equivariant():
    rng = _rng(10)
    q, k, v = (rng.standard_normal((12, 2, 8)) for _ in range(3))
    perm = rng.permutation(12)
    o = oracle.attention(q, k, v)
    op = oracle.attention(q[perm], k[perm], v[perm])
    np.testing.assert_allclose(op, o[perm], rtol=1e-12, atol=1e-14)


def test_attention_logits_shift_invariant():
    """q_i . k_j after the rotary depends only on the position difference."""
    rng = _rng(11)
    gh, gw, D = 4, 4, 64
    q = rng.standard_normal((gh * gw, 2, D))
    k = rng.standard_normal((gh * gw, 2, D))
    c0, s0 = oracle.rope_table(gh, gw, D)
    c1, s1 = oracle.rope_table(gh, gw, D, origin=(9, 23))
    l0 = np.einsum("phd,qhd->hpq", oracle.apply_rope(q, c0, s0), oracle.apply_rope(k, c0, s0))
    l1 = np.einsum("phd,qhd->hpq", oracle.apply_rope(q, c1, s1), oracle.apply_rope(k, c1, s1))
    np.testing.assert_allclose(l0, l1, rtol=1e-10, atol=1e-10)
    # and the probabilities through the oracle's softmax agree too
    a0 = oracle.attention_probs(oracle.apply_rope(q, c0, s0), oracle.apply_rope(k, c0, s0))
    a1 = oracle.attention_probs(oracle.apply_rope(q, c1, s1), oracle.apply_rope(k, c1, s1))
    np.testing.assert_allclose(a0, a1, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- MLP / block
def test_mlp_scalar_closed_form():
    x = np.array([[0.7]])
    a, b, c = 1.3, -0.4, 2.5
    z = a * 0.7
    expect = c * (z / (1 + math.exp(-z))) * (b * 0.7)
    got = oracle.mlp(x, np.array([[a]]), np.array([[b]]), np.array([[c]]))
    assert abs(got[0, 0] - expect) < 1e-15
    # swapping gate and up must change the answer (silu is not symmetric)
    swapped = oracle.mlp(x, np.array([[b]]), np.array([[a]]), np.array([[c]]))
    assert abs(swapped[0, 0] - expect) > 1e-3
    assert oracle.mlp(np.zeros((2, 3)), np.ones((4, 3)), np.ones((4, 3)), np.ones((3, 4))).max() == 0


def _tiny_weights(rng, d, h, n_blocks, L=0, std=0.3):
    def m(r, c):
        return rng.standard_normal((r, c)) * std
    w = {"patch_embed": m(d, 12), "blocks": []}
    for _ in range(n_blocks):
        w["blocks"].append({"norm1": 1 + 0.1 * rng.standard_normal(d), "wqkv": m(3 * d, d),
                            "wo": m(d, d), "norm2": 1 + 0.1 * rng.standard_normal(d),
                            "w_gate": m(h, d), "w_up": m(h, d), "w_down": m(d, h)})
    w["final_norm"] = 1 + 0.1 * rng.standard_normal(d)
    w["aligner"] = m(L, 4 * d) if L else None
    return w


def test_block_single_patch_closed_form():
    """One patch: attention returns v, so the block is x + Wo v + MLP(norm2(.))."""
    rng = _rng(12)
    d, h, H = 16, 24, 2
    w = _tiny_weights(rng, d, h, 1)["blocks"][0]
    x = rng.standard_normal((1, d))
    cos, sin = oracle.rope_table(1, 1, d // H)
    got = oracle.block(x, w, cos, sin, H)
    n1 = w["norm1"] * x / np.sqrt(np.mean(x * x) + 1e-6)
    v = n1 @ w["wqkv"][2 * d:3 * d].T  # the v rows are the last third of wqkv
    x1 = x + v @ w["wo"].T
    n2 = w["norm2"] * x1 / np.sqrt(np.mean(x1 * x1) + 1e-6)
    g, u = n2 @ w["w_gate"].T, n2 @ w["w_up"].T
    x2 = x1 + (g / (1 + np.exp(-g)) * u) @ w["w_down"].T
    np.testing.assert_allclose(got, x2, rtol=1e-12)


def test_tower_zero_branches_reduce_to_norm_of_embed():
    rng = _rng(13)
    d, h, H = 16, 24, 2
    w = _tiny_weights(rng, d, h, 3)
    for b in w["blocks"]:
        b["wo"][:] = 0
        b["w_down"][:] = 0
    X = rng.standard_normal((12, 12))
    got = oracle.tower(X, 3, 4, w, H)
    e = X @ w["patch_embed"].T
    expect = w["final_norm"] * e / np.sqrt(np.mean(e * e, -1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(got, expect, rtol=1e-12)


def _brute_encode(X, gh, gw, w, H, with_aligner):
    """Scalar-loop encoder written straight from the definitions (tiny sizes only)."""
    P = gh * gw
    d = len(w["final_norm"])
    D = d // H
    qd = D // 4
    theta = 10000.0

    def lin(vec, W):
        return [sum(vec[k] * W[n][k] for k in range(len(vec))) for n in range(len(W))]

    def rms(vec, sc):
        m = sum(t * t for t in vec) / len(vec)
        return [sc[i] * vec[i] / math.sqrt(m + 1e-6) for i in range(len(vec))]

    def rot(vec, r, c):
        out = list(vec)
        for hh in range(H):
            base = hh * D
            for half, pos in ((0, r), (1, c)):
                lo = base + half * (D // 2)
                for kk in range(qd):
                    ang = pos * theta ** (-kk / qd)
                    a1, a2 = vec[lo + kk], vec[lo + qd + kk]
                    out[lo + kk] = a1 * math.cos(ang) - a2 * math.sin(ang)
                    out[lo + qd + kk] = a2 * math.cos(ang) + a1 * math.sin(ang)
        return out

    x = [lin(list(X[p]), w["patch_embed"]) for p in range(P)]
    for b in w["blocks"]:
        qs, ks, vs = [], [], []
        for p in range(P):
            qkv = lin(rms(x[p], b["norm1"]), b["wqkv"])
            r, c = divmod(p, gw)
            qs.append(rot(qkv[0:d], r, c))
            ks.append(rot(qkv[d:2 * d], r, c))
            vs.append(qkv[2 * d:3 * d])
        att = [[0.0] * d for _ in range(P)]
        for hh in range(H):
            for i in range(P):
                lg = [sum(qs[i][hh * D + e] * ks[j][hh * D + e] for e in range(D)) / math.sqrt(D)
                      for j in range(P)]
                m = max(lg)
                ex = [math.exp(t - m) for t in lg]
                s = sum(ex)
                for j in range(P):
                    for e in range(D):
                        att[i][hh * D + e] += ex[j] / s * vs[j][hh * D + e]
        x = [[x[p][i] + t for i, t in enumerate(lin(att[p], b["wo"]))] for p in range(P)]
        nx = []
        for p in range(P):
            n2 = rms(x[p], b["norm2"])
            g, u = lin(n2, b["w_gate"]), lin(n2, b["w_up"])
            a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(len(g))]
            nx.append([x[p][i] + t for i, t in enumerate(lin(a, b["w_down"]))])
        x = nx
    x = [rms(x[p], w["final_norm"]) for p in range(P)]
    if not with_aligner:
        return np.array(x)
    out = []
    for i in range(gh // 2):
        for j in range(gw // 2):
            cat = []
            for a in range(2):
                for bb in range(2):
                    cat += x[(2 * i + a) * gw + 2 * j + bb]
            out.append(lin(cat, w["aligner"]))
    return np.array(out)


def test_encode_matches_scalar_brute_force():
    rng = _rng(14)
    d, h, H, L = 16, 20, 2, 5
    w = _tiny_weights(rng, d, h, 2, L)
    gh, gw = 2, 4
    X = rng.standard_normal((gh * gw, 12))
    got = oracle.encode(X, gh, gw, w, H, with_aligner=True)
    np.testing.assert_allclose(got, _brute_encode(X, gh, gw, w, H, True), rtol=1e-10, atol=1e-12)
    got = oracle.encode(X, gh, gw, w, H, with_aligner=False)
    np.testing.assert_allclose(got, _brute_encode(X, gh, gw, w, H, False), rtol=1e-10, atol=1e-12)


def test_varlen_images_do_not_see_each_other():
    rng = _rng(15)
    d, h, H = 16, 20, 2
    w = _tiny_weights(rng, d, h, 2)
    grids = [(2, 3), (3, 2), (1, 5)]
    X = rng.standard_normal((6 + 6 + 5, 12))
    a = oracle.encode_varlen(X, grids, w, H, with_aligner=False)
    X2 = X.copy()
    X2[6:12] = rng.standard_normal((6, 12))  # change only the second image
    b = oracle.encode_varlen(X2, grids, w, H, with_aligner=False)
    np.testing.assert_array_equal(a[:6], b[:6])
    np.testing.assert_array_equal(a[12:], b[12:])
    assert not np.allclose(a[6:12], b[6:12])
    # and the first image alone is exactly the first slice
    np.testing.assert_array_equal(a[:6], oracle.encode(X[:6], 2, 3, w, H, with_aligner=False))


def test_varlen_positions_restart_per_image():
    """Two identical images in one batch give identical outputs."""
    rng = _rng(16)
    d, h, H = 16, 20, 2
    w = _tiny_weights(rng, d, h, 1)
    X = rng.standard_normal((6, 12))
    out = oracle.encode_varlen(np.concatenate([X, X]), [(2, 3), (2, 3)], w, H, with_aligner=False)
    np.testing.assert_array_equal(out[:6], out[6:])


# ---------------------------------------------------------------- aligner layout
def _read_layout_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "aligner_layout_4x6.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *nums = line.split()
            vals[key] = np.array([int(t) for t in nums], dtype=np.int32)
    return vals


def test_aligner_perm_and_nlayout_golden():
    g = _read_layout_golden()
    np.testing.assert_array_equal(oracle.aligner_perm(4, 6), g["perm"])
    t, s = oracle.nlayout(4, 6)
    np.testing.assert_array_equal(t, g["nl_type"])
    np.testing.assert_array_equal(s, g["nl_src"])


@pytest.mark.parametrize("grid", [(2, 2), (28, 28), (64, 64), (48, 48), (10, 78), (6, 112)])
def test_aligner_perm_bijection_and_reshape_enumeration(grid):
    gh, gw = grid
    perm = oracle.aligner_perm(gh, gw)
    assert perm.dtype == np.int32
    assert np.array_equal(np.sort(perm), np.arange(gh * gw))
    # independent enumeration: view the index grid as (gh/2, 2, gw/2, 2) blocks
    idx = np.arange(gh * gw).reshape(gh // 2, 2, gw // 2, 2).transpose(0, 2, 1, 3).reshape(-1)
    np.testing.assert_array_equal(perm, idx)
    t, s = oracle.nlayout(gh, gw)
    hh, ww = gh // 2, gw // 2
    assert len(t) == hh * (ww + 1) + 2
    assert (t == 1).sum() == hh * ww and (t == 2).sum() == hh
    np.testing.assert_array_equal(s[t == 1], np.arange(hh * ww))
    assert (s[t != 1] == -1).all()


def test_aligner_identity_selector_gives_gather():
    rng = _rng(17)
    gh, gw, d = 4, 6, 3
    x = rng.standard_normal((gh * gw, d))
    G = oracle.aligner_gather(x, gh, gw)
    np.testing.assert_array_equal(oracle.aligner(x, gh, gw, np.eye(4 * d)), G)
    # merged token 4 = group (1, 1): patches (2,2) (2,3) (3,2) (3,3)
    np.testing.assert_array_equal(G[4], np.concatenate([x[14], x[15], x[20], x[21]]))


def test_aligner_rejects_odd_grid():
    with pytest.raises(ValueError):
        oracle.aligner_perm(27, 37)


# ---------------------------------------------------------------- synthetic inputs
def test_bf16_rounding_is_round_to_nearest_even():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5e-3], dtype=np.float32)
    r = synth.round_to_bf16(a)
    assert r[0] == 1.0
    assert r[1] == 1.0  # exact tie -> even (mantissa 0)
    assert r[2] == 1.0 + 4 * 2 ** -8  # tie -> even (up)
    assert r[3] == 1.0
    assert (r.view(np.uint32) & 0xFFFF == 0).all()


def test_synth_is_deterministic():
    from vision_transformer_encoder_image_amd import configs
    a = synth.make_inputs(configs.get(0), 0)
    b = synth.make_inputs(configs.get(0), 0)
    np.testing.assert_array_equal(a["patches"], b["patches"])
    np.testing.assert_array_equal(a["weights"]["blocks"][1]["w_down"], b["weights"]["blocks"][1]["w_down"])
    assert a["patches"].shape == (64, 588)
    assert a["weights"]["aligner"].shape == (512, 1024)


# ---------------------------------------------------------------- image-embedding merge
def _merge_fixture():
    types, expected = None, []
    for line in open(os.path.join(GOLDEN, "merge_embeddings_small.txt")):
        if line.startswith("types"):
            types = np.array([int(v) for v in line.split()[1:]], dtype=np.int32)
        elif line.startswith("expected"):
            expected.append([float(v) for v in line.split()[1:]])
    return types, np.array(expected)


def test_merge_embeddings_golden():
    types, expected = _merge_fixture()
    q = np.arange(len(types))
    embeds = np.stack([100.0 + q, -q.astype(float)], axis=1).reshape(2, 9, 2)
    tokens = np.stack([1000.0 + np.arange(5), 2000.0 + np.arange(5)], axis=1)
    sentinels = np.array([[7.0, 7.0], [8.0, 8.0], [9.0, 9.0]])
    got = oracle.merge_image_embeddings(embeds, types.reshape(2, 9), tokens, sentinels)
    assert got.shape == (2, 9, 2)
    np.testing.assert_array_equal(got.reshape(-1, 2), expected)


def test_merge_embeddings_with_nlayout_places_tokens_in_order():
    # two images laid out with the newline layout inside a text stream: every IMAGE slot
    # receives the aligned token its nl_src names (offset by the image's first token)
    rng = np.random.default_rng(3)
    L = 6
    spans, tok_off, src_all = [], 0, []
    for gh, gw in [(4, 6), (2, 8)]:
        t, src = oracle.nlayout(gh, gw)
        spans.append(t)
        src_all.append(np.where(src >= 0, src + tok_off, -1))
        tok_off += (gh // 2) * (gw // 2)
    text = np.full(5, -1, np.int32)
    types = np.concatenate([text, spans[0], text[:3], spans[1], text[:2]])
    srcs = np.concatenate([np.full(5, -1), src_all[0], np.full(3, -1), src_all[1], np.full(2, -1)])
    embeds = rng.standard_normal((len(types), L))
    tokens = rng.standard_normal((tok_off, L))
    sentinels = rng.standard_normal((3, L))
    got = oracle.merge_image_embeddings(embeds, types, tokens, sentinels)
    for q in range(len(types)):
        if types[q] == oracle.NL_IMAGE:
            np.testing.assert_array_equal(got[q], tokens[srcs[q]])
        elif types[q] == -1:
            np.testing.assert_array_equal(got[q], embeds[q])
        else:
            np.testing.assert_array_equal(got[q], sentinels[[oracle.NL_START, oracle.NL_NEWLINE,
                                                             oracle.NL_END].index(types[q])])
    # every token consumed exactly once
    assert (types == oracle.NL_IMAGE).sum() == tok_off


# ---------------------------------------------------------------- PatchMerger projector
def _ln_gelu_fixture():
    ln, ge = [], []
    for line in open(os.path.join(GOLDEN, "layernorm_gelu_small.txt")):
        if line.startswith("layernorm"):
            parts = [list(map(float, p.split())) for p in line[len("layernorm"):].split("|")]
            ln.append((np.array(parts[0]), np.array(parts[1]), np.array(parts[2]), parts[3][0],
                       np.array(parts[4])))
        elif line.startswith("gelu"):
            x, y = map(float, line.split()[1:])
            ge.append((x, y))
    return ln, ge


def test_layernorm_golden():
    ln, _ = _ln_gelu_fixture()
    assert len(ln) == 3
    for x, w, b, eps, want in ln:
        np.testing.assert_allclose(oracle.layernorm(x, w, b, eps), want, rtol=1e-14, atol=1e-14)


def test_layernorm_shift_scale_invariance_and_moments():
    rng = _rng(31)
    x = rng.standard_normal((5, 16))
    one, zero = np.ones(16), np.zeros(16)
    y = oracle.layernorm(x, one, zero, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.layernorm(3.5 * x - 2.0, one, zero, eps=0.0), y, rtol=1e-12,
                               atol=1e-12)
    w, b = rng.standard_normal(16), rng.standard_normal(16)
    np.testing.assert_allclose(oracle.layernorm(x, w, b, eps=0.0), y * w + b, rtol=1e-13, atol=1e-13)


def test_gelu_golden_and_odd_identity():
    _, ge = _ln_gelu_fixture()
    assert len(ge) == 7
    for x, want in ge:
        assert abs(float(oracle.gelu(np.array([x]))[0]) - want) < 1e-14
    x = np.linspace(-6, 6, 97)
    # x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=1e-13, atol=1e-13)


def test_patch_merger_param_count_is_the_pages():
    # the projector of the NVFP4 model page: 2x2 groups of 1152-dim patches, 4608 -> 4096
    assert oracle.patch_merger_param_count(1152, 4608, 4096) == 40_119_040
    # the count needs both norm parameters and both biases
    assert oracle.patch_merger_param_count(1152, 4608, 4096) - 1152 != 40_119_040


def test_patch_merger_scalar_loops():
    """Whole projector by scalar loops on a 2x4 grid: each patch (r, c) goes to merged
    token (r//2)*(gw//2) + c//2, slot 2*(r%2) + c%2 (placed directly, not through the
    gather of the oracle)."""
    rng = _rng(32)
    gh, gw, d, hid, out = 2, 4, 3, 5, 2
    x = rng.standard_normal((gh * gw, d))
    p = {"ln_w": rng.standard_normal(d), "ln_b": rng.standard_normal(d),
         "w1": rng.standard_normal((hid, 4 * d)), "b1": rng.standard_normal(hid),
         "w2": rng.standard_normal((out, hid)), "b2": rng.standard_normal(out)}
    eps = 1e-6
    T = gh * gw // 4
    g = [[0.0] * (4 * d) for _ in range(T)]
    for r in range(gh):
        for c in range(gw):
            row = x[r * gw + c]
            mu = sum(row) / d
            var = sum((v - mu) ** 2 for v in row) / d
            t, s = (r // 2) * (gw // 2) + c // 2, 2 * (r % 2) + c % 2
            for k in range(d):
                g[t][s * d + k] = (row[k] - mu) / math.sqrt(var + eps) * p["ln_w"][k] + p["ln_b"][k]
    want = np.zeros((T, out))
    for t in range(T):
        h = []
        for j in range(hid):
            a = p["b1"][j] + sum(p["w1"][j][k] * g[t][k] for k in range(4 * d))
            h.append(0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0))))
        for o in range(out):
            want[t, o] = p["b2"][o] + sum(p["w2"][o][j] * h[j] for j in range(hid))
    np.testing.assert_allclose(oracle.patch_merger(x, gh, gw, p, eps), want, rtol=1e-12, atol=1e-12)


def test_patch_merger_constant_patches_closed_form():
    """Constant patches normalise to the norm bias, so every merged token is
    W2 gelu(W1 [b, b, b, b] + b1) + b2."""
    rng = _rng(33)
    d, hid, out = 4, 6, 3
    p = {"ln_w": rng.standard_normal(d), "ln_b": rng.standard_normal(d),
         "w1": rng.standard_normal((hid, 4 * d)), "b1": rng.standard_normal(hid),
         "w2": rng.standard_normal((out, hid)), "b2": rng.standard_normal(out)}
    x = np.full((4 * 6, d), 2.5)
    a = p["w1"] @ np.tile(p["ln_b"], 4) + p["b1"]
    h = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in a])
    want = p["w2"] @ h + p["b2"]
    got = oracle.patch_merger(x, 4, 6, p)
    assert got.shape == (6, out)
    np.testing.assert_allclose(got, np.tile(want, (6, 1)), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- odd grids (zero padding)
def test_aligner_pad_odd_golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "aligner_pad_3x3.txt")):
        if line and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = np.array([int(t) for t in v], dtype=np.int32)
    np.testing.assert_array_equal(oracle.aligner_perm(3, 3, pad_odd=True), vals["perm"])
    types, src = oracle.nlayout(3, 3, pad_odd=True)
    np.testing.assert_array_equal(types, vals["types"])
    np.testing.assert_array_equal(src, vals["src"])
    with pytest.raises(ValueError):
        oracle.aligner_perm(3, 3)


@pytest.mark.parametrize("grid", [(3, 5), (4, 7), (5, 2), (1, 1), (6, 4)])
def test_aligner_pad_equals_explicit_zero_padding(grid):
    """The padded merge of an odd grid equals the plain merge of the grid padded by
    hand with zero patches (and is the plain merge on even grids)."""
    gh, gw = grid
    rng = _rng(34)
    d = 3
    x = rng.standard_normal((gh * gw, d))
    ph, pw = gh + gh % 2, gw + gw % 2
    xp = np.zeros((ph, pw, d))
    xp[:gh, :gw] = x.reshape(gh, gw, d)
    want = oracle.aligner_gather(xp.reshape(ph * pw, d), ph, pw)
    np.testing.assert_array_equal(oracle.aligner_gather(x, gh, gw, pad_odd=True), want)
    types, _ = oracle.nlayout(gh, gw, pad_odd=True)
    assert (types == oracle.NL_IMAGE).sum() == want.shape[0] == (ph // 2) * (pw // 2)


# ---------------------------------------------------------------- MLP half backward
def test_mlp_half_backward_matches_finite_differences():
    """Central differences of L = sum(dy * (x + mlp(rmsnorm(x, w)))) built from the
    pinned forward steps, for every input of the MLP half."""
    rng = _rng(35)
    P, d, h = 3, 4, 5
    x = rng.standard_normal((P, d))
    w = 1.0 + 0.3 * rng.standard_normal(d)
    wg, wu = rng.standard_normal((h, d)), rng.standard_normal((h, d))
    wd = rng.standard_normal((d, h))
    dy = rng.standard_normal((P, d))
    eps = 1e-3

    def loss(x_, w_, wg_, wu_, wd_):
        y = x_ + oracle.mlp(oracle.rmsnorm(x_, w_, eps), wg_, wu_, wd_)
        return float(np.sum(dy * y))

    grads = oracle.mlp_half_backward(x, w, wg, wu, wd, dy, eps)
    args = [x, w, wg, wu, wd]
    step = 1e-6
    for k, (arg, grad) in enumerate(zip(args, grads)):
        assert grad.shape == arg.shape
        fd = np.zeros_like(arg)
        for idx in np.ndindex(arg.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[k][idx] += step
            minus[k][idx] -= step
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * step)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"input {k}")


def test_mlp_half_backward_zero_branch_passes_dy():
    """With W_down = 0 the branch is constant zero: dx = dy, and only dW_down is non-zero
    (it equals dy^T a)."""
    rng = _rng(36)
    P, d, h = 5, 8, 6
    x = rng.standard_normal((P, d))
    w = np.ones(d)
    wg, wu = rng.standard_normal((h, d)), rng.standard_normal((h, d))
    dy = rng.standard_normal((P, d))
    dx, dw, dwg, dwu, dwd = oracle.mlp_half_backward(x, w, wg, wu, np.zeros((d, h)), dy)
    np.testing.assert_array_equal(dx, dy)
    assert not dw.any() and not dwg.any() and not dwu.any()
    n = oracle.rmsnorm(x, w)
    g, u = n @ wg.T, n @ wu.T
    np.testing.assert_allclose(dwd, dy.T @ (g / (1 + np.exp(-g)) * u), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("D", [4, 12])
def test_attn_half_backward_matches_finite_differences(D):
    """Central differences of L = sum(dy * (x + attn(norm1(x)))) built from the pinned
    forward steps (rmsnorm, linear, apply_rope, attention) on a 2x3 grid, 2 heads; head
    dims 4 and 12 (one and three rotated pairs per quarter; the 1152-wide tower has 18)."""
    rng = _rng(37 + D)
    gh, gw, H = 2, 3, 2
    P, d = gh * gw, H * D
    x = rng.standard_normal((P, d))
    w = 1.0 + 0.3 * rng.standard_normal(d)
    wqkv = 0.5 * rng.standard_normal((3 * d, d))
    wo = rng.standard_normal((d, d))
    dy = rng.standard_normal((P, d))
    cos, sin = oracle.rope_table(gh, gw, D, 10000.0)
    eps = 1e-3

    def loss(x_, w_, wqkv_, wo_):
        n = oracle.rmsnorm(x_, w_, eps)
        qkv = oracle.linear(n, wqkv_)
        q = oracle.apply_rope(qkv[:, :d].reshape(P, H, D), cos, sin)
        k = oracle.apply_rope(qkv[:, d:2 * d].reshape(P, H, D), cos, sin)
        v = qkv[:, 2 * d:].reshape(P, H, D)
        o = oracle.attention(q, k, v).reshape(P, d)
        return float(np.sum(dy * (x_ + oracle.linear(o, wo_))))

    grads = oracle.attn_half_backward(x, w, wqkv, wo, cos, sin, H, dy, eps)
    args = [x, w, wqkv, wo]
    step = 1e-6
    for k_, (arg, grad) in enumerate(zip(args, grads)):
        assert grad.shape == arg.shape
        fd = np.zeros_like(arg)
        for idx in np.ndindex(arg.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[k_][idx] += step
            minus[k_][idx] -= step
            fd[idx] = (loss(*plus) - loss(*minus)) / (2 * step)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"input {k_}")


def _fd_check(loss, args, grads, rng=None, max_entries=None, rtol=1e-6, atol=1e-7, tag=""):
    """Central differences of loss(*args) against the analytic grads (all entries,
    or max_entries random ones per argument)."""
    step = 1e-6
    for k_, (arg, grad) in enumerate(zip(args, grads)):
        assert grad.shape == arg.shape, (tag, k_)
        idxs = list(np.ndindex(arg.shape))
        if max_entries is not None and len(idxs) > max_entries:
            idxs = [idxs[i] for i in rng.choice(len(idxs), max_entries, replace=False)]
        for idx in idxs:
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[k_][idx] += step
            minus[k_][idx] -= step
            fd = (loss(*plus) - loss(*minus)) / (2 * step)
            np.testing.assert_allclose(grad[idx], fd, rtol=rtol, atol=atol,
                                       err_msg=f"{tag} argument {k_} entry {idx}")


def test_rmsnorm_backward_matches_finite_differences():
    """Central differences of L = sum(G * rmsnorm(x, w)) built from the pinned rmsnorm."""
    rng = _rng(41)
    x = rng.standard_normal((4, 8))
    w = 1.0 + 0.3 * rng.standard_normal(8)
    G = rng.standard_normal((4, 8))
    eps = 1e-3
    loss = lambda x_, w_: float(np.sum(G * oracle.rmsnorm(x_, w_, eps)))
    _fd_check(loss, [x, w], oracle.rmsnorm_backward(x, w, G, eps), tag="rmsnorm")


@pytest.mark.parametrize("n_blocks", [0, 2])
def test_tower_backward_matches_finite_differences(n_blocks):
    """Central differences of L = sum(G * tower outputs) with the pinned forward
    (encode_varlen without the aligner: patch embedding, blocks, final norm, one
    image at a time) on two ragged grids (2x3, 3x2), 2 heads of 4, every weight
    tensor (up to 12 random entries of each larger one)."""
    rng = _rng(42 + n_blocks)
    grids = [(2, 3), (3, 2)]
    H, D, hdn, pd = 2, 4, 12, 6
    d = H * D
    P = sum(a * b for a, b in grids)
    patches = rng.standard_normal((P, pd))
    G = rng.standard_normal((P, d))
    eps = 1e-3
    weights = {"patch_embed": 0.5 * rng.standard_normal((d, pd)),
               "final_norm": 1.0 + 0.3 * rng.standard_normal(d), "blocks": []}
    names = ["norm1", "wqkv", "wo", "norm2", "w_gate", "w_up", "w_down"]
    shapes = [(d,), (3 * d, d), (d, d), (d,), (hdn, d), (hdn, d), (d, hdn)]
    for _ in range(n_blocks):
        blk = {}
        for nm, sh in zip(names, shapes):
            blk[nm] = (1.0 + 0.3 * rng.standard_normal(sh)) if nm.startswith("norm") else \
                0.5 * rng.standard_normal(sh)
        weights["blocks"].append(blk)
    got = oracle.tower_backward(patches, grids, weights, H, G, eps)

    flat = [weights["patch_embed"], weights["final_norm"]] + \
        [blk[nm] for blk in weights["blocks"] for nm in names]
    grads = [got["patch_embed"], got["final_norm"]] + \
        [gb[nm] for gb in got["blocks"] for nm in names]

    def loss(*ws):
        w = {"patch_embed": ws[0], "final_norm": ws[1],
             "blocks": [dict(zip(names, ws[2 + 7 * b:9 + 7 * b])) for b in range(n_blocks)]}
        out = oracle.encode_varlen(patches, grids, w, H, eps, with_aligner=False)
        return float(np.sum(G * out))

    _fd_check(loss, flat, grads, rng=rng, max_entries=12, rtol=1e-5, atol=1e-7, tag="tower")
