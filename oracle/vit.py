"""Oracle steps of the vision encoder (test infrastructure only; see package doc).

Sources (web pages):
  [VIS]  NeMo Automodel API docs, ``nemo_automodel.components.models.deepseek_v4.vision``
         (classes DeepseekV4VisionPatchEmbed, RMSNorm, Attention, MLP, Block,
         Transformer, Aligner; functions apply_vision_rotary, get_vision_cos_sin).
  [MOD]  NeMo Automodel API docs, ``...deepseek_v4.model`` (DeepseekV4Model.encode_image,
         forward arguments ``pixel_values`` / ``image_grid_hws``; image sentinel
         parameters image_start / image_newline / image_pad / image_end).
  [PR]   NVIDIA-NeMo/Automodel PR #3772 (Changelog; Validation: vision-only parity
         table with grids and "N-layout" / "Permutation" columns).
  [HF]   summary page of the HF DeepSeek-V4-Flash-Vision-Exp text model (the
         ``rotate_half`` pattern computed in fp32 and cast back).
  [NVFP4] model page of DeepSeek-V4-Flash-Vision-NVFP4 (the PatchMerger projector:
         2x2 groups of 1152-dim MoonViT patches -> 4608 -> 4096, 40,119,040 parameters).
"""
from __future__ import annotations

import numpy as np

# Readings taken where the pages leave a step open (same list as the design notes).
READINGS = {
    "rope_freq": "each half of a head is a 1D rotary of width D/2 with f_k = theta^(-k/(D/4)), k < D/4",
    "rope_pairing": "rotate_half pairing inside each half: element i pairs with i + D/4",
    "rope_axes": "first D/2 dims rotated by the patch row index, last D/2 by the column index",
    "positions": "0-based integer (row, col) with p = row*gw + col, restarting for every image",
    "attention": "scale 1/sqrt(D), no mask inside an image, images never see each other",
    "wqkv": "rows ordered [q; k; v], each head-major (head h owns rows h*D .. h*D+D-1)",
    "bias": "no bias in patch embed, wqkv, out-proj, MLP or aligner",
    "rmsnorm": "y = w * x / sqrt(mean(x^2) + eps), eps inside the root, fp32 scale w",
    "final_norm": "applied once after the last block, before the aligner",
    "patch_order": "patch (r, c) flattens img[:, 14r:14r+14, 14c:14c+14] in C order [3,14,14]",
    "swiglu": "silu(x Wg^T) * (x Wu^T), then Wd; no clamp",
    "aligner": "2x2 groups row-major over (gh/2, gw/2); inside a group TL,TR,BL,BR concatenated "
               "along features; one bias-free linear to the LLM width",
    "odd_grid": "the released aligner handles odd grids ([PR] validation: 27x37, 37x27, 112x7 "
                "exact) by a rule the pages do not give; by default odd grids are rejected, and "
                "with pad_odd the grid is zero-padded to even (a zero patch row below, a zero "
                "patch column on the right) before the 2x2 merge, so an image has "
                "ceil(gh/2)*ceil(gw/2) merged tokens",
    "nlayout": "per image: [START] + per merged row (w' IMAGE, NEWLINE) + [END]; "
               "types START=0 IMAGE=1 NEWLINE=2 END=3; src = merged token index or -1",
    "merge_embeddings": "positions are visited batch-major, sequence-minor; IMAGE positions "
                        "take the aligned tokens in that order (the images' concatenation "
                        "order), START/NEWLINE/END take the image_start/image_newline/"
                        "image_end embeddings, -1 (text) and any other type stay as they are; "
                        "image_pad is not used by this layout",
    "patch_merger": "the 40,119,040 projector parameters decompose exactly as a norm over the "
                    "1152 patch features with weight and bias (2*1152), Linear(4608, 4608) with "
                    "bias and Linear(4608, 4096) with bias; so: LayerNorm (mean and variance "
                    "over the features, eps 1e-6 inside the root) on every patch, the aligner's "
                    "2x2 gather, the first linear, GELU in its erf form (the activation is not "
                    "named), the second linear",
}

NL_START, NL_IMAGE, NL_NEWLINE, NL_END = 0, 1, 2, 3


def _f(a, dtype):
    return np.asarray(a, dtype=dtype)


def linear(x, w, dtype=np.float64):
    """Bias-free linear map with a PyTorch-style weight ``[out, in]``: y = x W^T.

    [VIS] every projection (patch_embed.proj, wqkv, out-proj, MLP, aligner) is a
    linear map; the MLP page calls it bias-free and no bias is named elsewhere.
    """
    return _f(x, dtype) @ _f(w, dtype).T


def patchify(img, patch_size=14):
    """Cut a ``[3, gh*ps, gw*ps]`` image into ``[gh*gw, 3*ps*ps]`` row-major patches.

    [VIS] DeepseekV4VisionTransformer.forward takes patches ``[n_h*n_w, 3, ps, ps]``;
    patch p = r*gw + c holds pixels rows ps*r.., cols ps*c.. flattened in C order.
    """
    img = np.asarray(img)
    C, Hpx, Wpx = img.shape
    gh, gw = Hpx // patch_size, Wpx // patch_size
    out = np.empty((gh * gw, C * patch_size * patch_size), dtype=img.dtype)
    for r in range(gh):
        for c in range(gw):
            tile = img[:, r * patch_size:(r + 1) * patch_size, c * patch_size:(c + 1) * patch_size]
            out[r * gw + c] = tile.reshape(-1)
    return out


def patch_embed(patches, w, dtype=np.float64):
    """[VIS] DeepseekV4VisionPatchEmbed: project flattened RGB patches to vision_dim."""
    p = _f(patches, dtype).reshape(len(patches), -1)
    return linear(p, w, dtype)


def rmsnorm(x, w, eps=1e-6, dtype=np.float64):
    """[VIS] DeepseekV4VisionRMSNorm(dim, eps=1e-6) with an fp32 scale parameter.

    y = w * x / sqrt(mean(x^2 over the last axis) + eps).
    """
    x = _f(x, dtype)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f(w, dtype) * (x / np.sqrt(ms + eps))


def rope_freqs(head_dim, theta=10000.0):
    """Rotary frequencies of one half of a head (width D/2): f_k = theta^(-k/(D/4)).

    [VIS] apply_vision_rotary is a "half-split 2D" rotary whose tables have width
    head_dim/2; the theta is the transformer's ``rope_theta``.  Each half is read as
    a standard 1D rotary of width D/2 (reading "rope_freq").
    """
    q = head_dim // 4
    return np.array([theta ** (-(k / q)) for k in range(q)], dtype=np.float64)


def rope_table(gh, gw, head_dim, theta=10000.0, origin=(0, 0)):
    """Cos/sin tables ``[gh*gw, D/2]`` = [row-angle part D/4 | column-angle part D/4].

    [VIS] get_vision_cos_sin(n_h, n_w, dim, theta) builds the 2D table for one image;
    patch p sits at row p // gw and column p % gw.  ``origin`` shifts every position
    by the same offset (used only by the shift-invariance pin).  Built in float64.
    """
    f = rope_freqs(head_dim, theta)
    P = gh * gw
    cos = np.empty((P, head_dim // 2), dtype=np.float64)
    sin = np.empty((P, head_dim // 2), dtype=np.float64)
    q = head_dim // 4
    for p in range(P):
        r = p // gw + origin[0]
        c = p % gw + origin[1]
        cos[p, :q] = np.cos(r * f)
        sin[p, :q] = np.sin(r * f)
        cos[p, q:] = np.cos(c * f)
        sin[p, q:] = np.sin(c * f)
    return cos, sin


def apply_rope(x, cos, sin, dtype=np.float64):
    """Half-split 2D rotary on ``[P, H, D]``.

    [VIS] apply_vision_rotary: the first half A = x[:D/2] of each head rotates with
    the row angles, the second half B = x[D/2:] with the column angles.  Inside a
    half, [a1 | a2] (quarters) maps to [a1 cos - a2 sin | a2 cos + a1 sin], the
    rotate_half pattern ([HF]: x*cos + rotate_half(x)*sin with
    rotate_half([a1|a2]) = [-a2|a1]).
    """
    x = _f(x, dtype)
    P, H, D = x.shape
    q = D // 4
    out = np.empty_like(x)
    for half in range(2):
        lo = half * (D // 2)
        c = _f(cos[:, half * q:(half + 1) * q], dtype)[:, None, :]
        s = _f(sin[:, half * q:(half + 1) * q], dtype)[:, None, :]
        a1 = x[:, :, lo:lo + q]
        a2 = x[:, :, lo + q:lo + 2 * q]
        out[:, :, lo:lo + q] = a1 * c - a2 * s
        out[:, :, lo + q:lo + 2 * q] = a2 * c + a1 * s
    return out


def attention_probs(q, k, dtype=np.float64):
    """Softmax(Q K^T / sqrt(D)) per head for one image: ``[H, P, P]``.

    [VIS] DeepseekV4VisionAttention: full bidirectional patch attention over one
    image (no mask).  Scale 1/sqrt(head_dim) (reading "attention").
    """
    q = _f(q, dtype)
    k = _f(k, dtype)
    P, H, D = q.shape
    out = np.empty((H, P, k.shape[0]), dtype=dtype)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) / np.sqrt(D)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        out[h] = e / e.sum(axis=-1, keepdims=True)
    return out


def attention(q, k, v, dtype=np.float64):
    """O = softmax(Q K^T / sqrt(D)) V per head for one image; ``[P, H, D]``.

    One head at a time (same arithmetic as ``attention_probs``, less memory).
    """
    q, k, v = _f(q, dtype), _f(k, dtype), _f(v, dtype)
    out = np.empty_like(v)
    for h in range(q.shape[1]):
        a = attention_probs(q[:, h:h + 1], k[:, h:h + 1], dtype)[0]
        out[:, h, :] = a @ v[:, h, :]
    return out


def mlp(x, w_gate, w_up, w_down, dtype=np.float64):
    """[VIS] DeepseekV4VisionMLP: bias-free SwiGLU, silu(x Wg^T) * (x Wu^T), then Wd."""
    g = linear(x, w_gate, dtype)
    u = linear(x, w_up, dtype)
    return linear((g / (1.0 + np.exp(-g))) * u, w_down, dtype)


def mlp_half_backward(x, norm_w, w_gate, w_up, w_down, dy, eps=1e-6, dtype=np.float64):
    """Gradients of the MLP half of a block ([VIS] DeepseekV4VisionBlock's second
    residual branch, y = x + mlp(norm2(x)); [PR] lists backward over ragged grids
    among the tested paths): given dy = dL/dy, returns dL/d(x, norm_w, w_gate,
    w_up, w_down) by the chain rule through the steps of ``rmsnorm`` and ``mlp``.

    With r = (mean(x^2) + eps)^-1/2, n = norm_w * x * r, g = n Wg^T, u = n Wu^T,
    s = sigmoid(g), a = g s u:
      da = dy Wd,  dWd = dy^T a,
      dg = da u (s + g s (1 - s)),  du = da g s,
      dn = dg Wg + du Wu,  dWg = dg^T n,  dWu = du^T n,
      d norm_w = sum over rows of dn x r,
      dx = dy + r (norm_w dn) - x r^3 mean(norm_w dn x).
    """
    x, dy = _f(x, dtype), _f(dy, dtype)
    w, wg, wu, wd = (_f(a, dtype) for a in (norm_w, w_gate, w_up, w_down))
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = w * x * r
    g, u = n @ wg.T, n @ wu.T
    sg = 1.0 / (1.0 + np.exp(-g))
    a = g * sg * u
    da = dy @ wd
    d_wd = dy.T @ a
    dg = da * u * (sg + g * sg * (1.0 - sg))
    du = da * g * sg
    dn = dg @ wg + du @ wu
    d_wg, d_wu = dg.T @ n, du.T @ n
    d_w = np.sum(dn * x * r, axis=0)
    wdn = w * dn
    dx = dy + r * wdn - x * r ** 3 * np.mean(wdn * x, axis=-1, keepdims=True)
    return dx, d_w, d_wg, d_wu, d_wd


def attn_half_backward(x, norm_w, wqkv, wo, cos, sin, n_heads, dy, eps=1e-6, dtype=np.float64):
    """Gradients of the attention half of a block for one image ([VIS]
    DeepseekV4VisionBlock's first residual branch, y = x + attn(norm1(x)) with the
    steps of ``block``; reading "backward"): given dy, returns dL/d(x, norm_w,
    wqkv, wo) by the chain rule.

    With n = norm1(x), [q|k|v] = n Wqkv^T, q', k' the rotated q, k, per head
    P = softmax(q' k'^T / sqrt(D)) and o = P v:
      do = dy Wo,  dWo = dy^T o,
      dv = P^T do,  dP = do v^T,  dS = P (dP - rowsum(dP P)),
      dq' = dS k' / sqrt(D),  dk' = dS^T q' / sqrt(D),
      dq, dk = the rotary applied with the opposite angles (its transpose),
      dn = [dq|dk|dv] Wqkv,  dWqkv = [dq|dk|dv]^T n,
      then the RMSNorm gradient as in ``mlp_half_backward``, plus dy.
    """
    x, dy = _f(x, dtype), _f(dy, dtype)
    w, wqkv, wo = _f(norm_w, dtype), _f(wqkv, dtype), _f(wo, dtype)
    P, d = x.shape
    D = d // n_heads
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = w * x * r
    qkv = n @ wqkv.T
    q = apply_rope(qkv[:, 0:d].reshape(P, n_heads, D), cos, sin, dtype)
    k = apply_rope(qkv[:, d:2 * d].reshape(P, n_heads, D), cos, sin, dtype)
    v = qkv[:, 2 * d:].reshape(P, n_heads, D)
    probs = attention_probs(q, k, dtype)                    # [H, P, P]
    o = np.stack([probs[h] @ v[:, h] for h in range(n_heads)], axis=1).reshape(P, d)
    do = (dy @ wo).reshape(P, n_heads, D)
    d_wo = dy.T @ o
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for h in range(n_heads):
        p_h = probs[h]                                      # [queries, keys]
        dv[:, h] = p_h.T @ do[:, h]
        dp = do[:, h] @ v[:, h].T
        ds = p_h * (dp - np.sum(dp * p_h, axis=-1, keepdims=True))
        dq[:, h] = ds @ k[:, h] / np.sqrt(D)
        dk[:, h] = ds.T @ q[:, h] / np.sqrt(D)
    dq = apply_rope(dq, cos, -np.asarray(sin), dtype)
    dk = apply_rope(dk, cos, -np.asarray(sin), dtype)
    dqkv = np.concatenate([dq.reshape(P, d), dk.reshape(P, d), dv.reshape(P, d)], axis=1)
    d_wqkv = dqkv.T @ n
    dn = dqkv @ wqkv
    d_w = np.sum(dn * x * r, axis=0)
    wdn = w * dn
    dx = dy + r * wdn - x * r ** 3 * np.mean(wdn * x, axis=-1, keepdims=True)
    return dx, d_w, d_wqkv, d_wo


def rmsnorm_backward(x, norm_w, dy, eps=1e-6, dtype=np.float64):
    """Gradients of y = rmsnorm(x, norm_w) ([VIS] DeepseekV4VisionRMSNorm) for dy:
    with r = (mean(x^2) + eps)^-1/2 and g = norm_w dy,
      dx = r g - x r^3 mean(g x),  d norm_w = sum over rows of dy x r."""
    x, dy, w = _f(x, dtype), _f(dy, dtype), _f(norm_w, dtype)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = w * dy
    dx = r * g - x * r ** 3 * np.mean(g * x, axis=-1, keepdims=True)
    return dx, np.sum(dy * x * r, axis=0)


def _attn_branch(x, blk, cos, sin, n_heads, eps, dtype):
    """x + attn(norm1(x)) for one image: the first residual branch of ``block``."""
    P, d = x.shape
    D = d // n_heads
    n = rmsnorm(x, blk["norm1"], eps, dtype)
    qkv = linear(n, blk["wqkv"], dtype)
    q = apply_rope(qkv[:, 0:d].reshape(P, n_heads, D), cos, sin, dtype)
    k = apply_rope(qkv[:, d:2 * d].reshape(P, n_heads, D), cos, sin, dtype)
    v = qkv[:, 2 * d:3 * d].reshape(P, n_heads, D)
    return x + linear(attention(q, k, v, dtype).reshape(P, d), blk["wo"], dtype)


def tower_backward(patches, grids, weights, n_heads, dy, eps=1e-6, theta=10000.0,
                   dtype=np.float64):
    """Gradients of the tower ([VIS] DeepseekV4VisionTransformer.forward: patch
    embedding, blocks, final norm) over concatenated images, for dy = dL/d(output)
    ([PR] lists backward over ragged grids among the tested paths).

    The forward is run once with the residual stream kept at the input of every
    residual branch; then, in reverse, the final norm's gradient, each block's MLP
    half (``mlp_half_backward``) and attention half (``attn_half_backward``, one
    image at a time, weight gradients summed over the images), and last the patch
    embedding's weight gradient dWpe = dx0^T patches.  Returns a dict with
    ``patch_embed``, ``final_norm`` and ``blocks`` (per block ``norm1``, ``wqkv``,
    ``wo``, ``norm2``, ``w_gate``, ``w_up``, ``w_down``)."""
    patches, dy = _f(patches, dtype), _f(dy, dtype)
    x = patch_embed(patches, weights["patch_embed"], dtype)
    d = x.shape[1]
    spans, tables, off = [], [], 0
    for gh, gw in grids:
        spans.append(slice(off, off + gh * gw))
        tables.append(rope_table(gh, gw, d // n_heads, theta))
        off += gh * gw
    saved = []
    for blk in weights["blocks"]:
        xm = np.empty_like(x)
        for sl, (cos, sin) in zip(spans, tables):
            xm[sl] = _attn_branch(x[sl], blk, cos, sin, n_heads, eps, dtype)
        saved.append((x, xm))
        x = xm + mlp(rmsnorm(xm, blk["norm2"], eps, dtype), blk["w_gate"], blk["w_up"],
                     blk["w_down"], dtype)
    dx, d_final = rmsnorm_backward(x, weights["final_norm"], dy, eps, dtype)
    grads = []
    for blk, (xa, xm) in zip(reversed(weights["blocks"]), reversed(saved)):
        dx, d_n2, d_wg, d_wu, d_wd = mlp_half_backward(xm, blk["norm2"], blk["w_gate"],
                                                       blk["w_up"], blk["w_down"], dx, eps, dtype)
        dxa = np.empty_like(dx)
        d_n1, d_wqkv, d_wo = 0.0, 0.0, 0.0
        for sl, (cos, sin) in zip(spans, tables):
            r = attn_half_backward(xa[sl], blk["norm1"], blk["wqkv"], blk["wo"], cos, sin,
                                   n_heads, dx[sl], eps, dtype)
            dxa[sl] = r[0]
            d_n1, d_wqkv, d_wo = d_n1 + r[1], d_wqkv + r[2], d_wo + r[3]
        dx = dxa
        grads.append({"norm1": d_n1, "wqkv": d_wqkv, "wo": d_wo, "norm2": d_n2,
                      "w_gate": d_wg, "w_up": d_wu, "w_down": d_wd})
    return {"patch_embed": dx.T @ patches, "final_norm": d_final, "blocks": grads[::-1]}


def block(x, blk, cos, sin, n_heads, eps=1e-6, dtype=np.float64):
    """[VIS] DeepseekV4VisionBlock: x += attn(norm1(x)); x += mlp(norm2(x)).

    Inside attn ([VIS] DeepseekV4VisionAttention): wqkv -> q, k, v ``[P, H, D]``,
    rotary on q and k, full attention, out-projection ``wo``.
    """
    x = _f(x, dtype)
    P, d = x.shape
    D = d // n_heads
    n = rmsnorm(x, blk["norm1"], eps, dtype)
    qkv = linear(n, blk["wqkv"], dtype)
    q = qkv[:, 0:d].reshape(P, n_heads, D)
    k = qkv[:, d:2 * d].reshape(P, n_heads, D)
    v = qkv[:, 2 * d:3 * d].reshape(P, n_heads, D)
    q = apply_rope(q, cos, sin, dtype)
    k = apply_rope(k, cos, sin, dtype)
    o = attention(q, k, v, dtype).reshape(P, d)
    x = x + linear(o, blk["wo"], dtype)
    n2 = rmsnorm(x, blk["norm2"], eps, dtype)
    return x + mlp(n2, blk["w_gate"], blk["w_up"], blk["w_down"], dtype)


def tower(patches, gh, gw, weights, n_heads, eps=1e-6, theta=10000.0, dtype=np.float64,
          origin=(0, 0)):
    """[VIS] DeepseekV4VisionTransformer.forward for one image: embed, blocks, final norm."""
    x = patch_embed(patches, weights["patch_embed"], dtype)
    d = x.shape[1]
    cos, sin = rope_table(gh, gw, d // n_heads, theta, origin)
    for blk in weights["blocks"]:
        x = block(x, blk, cos, sin, n_heads, eps, dtype)
    return rmsnorm(x, weights["final_norm"], eps, dtype)


def _merged_dims(gh, gw, merge, pad_odd):
    if gh % merge or gw % merge:
        if not pad_odd:
            raise ValueError("aligner needs a grid divisible by the merge size")
        return -(-gh // merge), -(-gw // merge)
    return gh // merge, gw // merge


def aligner_perm(gh, gw, merge=2, pad_odd=False):
    """Source patch of every slot of the merged layout, ``[4 * tokens]`` int32.

    [VIS] DeepseekV4VisionAligner spatially downsamples (downsample_ratio = 2) and
    [PR] reports the permutation as exact; reading "aligner": merged token
    t = i*(w') + j gathers the 2x2 group at rows 2i..2i+1, cols 2j..2j+1 in
    row-major order TL, TR, BL, BR.  Reading "odd_grid": with ``pad_odd`` a slot
    outside the grid (row gh or column gw of the padded grid) holds -1.
    """
    hq, wq = _merged_dims(gh, gw, merge, pad_odd)
    perm = []
    for i in range(hq):
        for j in range(wq):
            for a in range(merge):
                for b in range(merge):
                    r, c = merge * i + a, merge * j + b
                    perm.append(r * gw + c if r < gh and c < gw else -1)
    return np.array(perm, dtype=np.int32)


def aligner_gather(x, gh, gw, merge=2, pad_odd=False):
    """G[t] = concat of x over the group of merged token t: ``[tokens, 4d]``
    (zero rows for the padded slots of an odd grid)."""
    x = np.asarray(x)
    perm = aligner_perm(gh, gw, merge, pad_odd)
    m2 = merge * merge
    rows = np.zeros((len(perm), x.shape[1]), dtype=x.dtype)
    rows[perm >= 0] = x[perm[perm >= 0]]
    return rows.reshape(len(perm) // m2, m2 * x.shape[1])


def aligner(x, gh, gw, w, merge=2, dtype=np.float64, pad_odd=False):
    """[VIS] DeepseekV4VisionAligner.forward: 2x2 gather, then the linear map to LLM width."""
    return linear(aligner_gather(_f(x, dtype), gh, gw, merge, pad_odd), w, dtype)


def layernorm(x, w, b, eps=1e-6, dtype=np.float64):
    """Norm of the PatchMerger projector ([NVFP4]), reading "patch_merger":
    y = (x - mean(x)) / sqrt(var(x) + eps) * w + b over the last axis, with the
    population variance (mean of squared deviations)."""
    x = _f(x, dtype)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f(w, dtype) + _f(b, dtype)


def gelu(x, dtype=np.float64):
    """GELU in its erf form, x * Phi(x) = x/2 * (1 + erf(x / sqrt(2))) (reading
    "patch_merger": the projector's activation is not named on the pages)."""
    from scipy.special import erf

    x = _f(x, dtype)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def patch_merger(x, gh, gw, p, eps=1e-6, merge=2, dtype=np.float64):
    """[NVFP4] PatchMerger projector for one image, reading "patch_merger": LayerNorm
    on every patch of ``x`` ``[gh*gw, d]``, the 2x2 gather of the aligner (same group
    order), Linear(4d, hidden) + bias, GELU, Linear(hidden, out) + bias.  ``p`` holds
    ln_w, ln_b [d]; w1 [hidden, 4d], b1 [hidden]; w2 [out, hidden], b2 [out]."""
    n = layernorm(x, p["ln_w"], p["ln_b"], eps, dtype)
    g = aligner_gather(n, gh, gw, merge)
    h = gelu(linear(g, p["w1"], dtype) + _f(p["b1"], dtype), dtype)
    return linear(h, p["w2"], dtype) + _f(p["b2"], dtype)


def patch_merger_param_count(d, hidden, out, merge=2):
    """Parameters of the projector of ``patch_merger``: norm weight and bias, then
    the two biased linear maps."""
    m2 = merge * merge
    return 2 * d + hidden * m2 * d + hidden + out * hidden + out


def nlayout(gh, gw, merge=2, pad_odd=False):
    """Newline layout of one image span in the LLM stream: (types, src) int32.

    [PR] names the released "N-layout pseudo-token expansion"; [MOD] names the
    sentinels image_start / image_newline / image_end.  Reading "nlayout": the span
    is [START], then for each merged row i its gw/2 IMAGE tokens followed by one
    NEWLINE, then [END].  ``src`` holds the merged token index of IMAGE slots and
    -1 for sentinels.  With ``pad_odd`` the merged grid is ceil(gh/2) x ceil(gw/2).
    """
    hh, ww = _merged_dims(gh, gw, merge, pad_odd)
    types, src = [NL_START], [-1]
    t = 0
    for _ in range(hh):
        for _ in range(ww):
            types.append(NL_IMAGE)
            src.append(t)
            t += 1
        types.append(NL_NEWLINE)
        src.append(-1)
    types.append(NL_END)
    src.append(-1)
    return np.array(types, dtype=np.int32), np.array(src, dtype=np.int32)


def merge_image_embeddings(embeds, types, tokens, sentinels):
    """[MOD] DeepseekV4Model.merge_image_embeddings: replace pseudo-token embeddings.

    ``embeds`` [..., L] text embeddings (any leading shape, e.g. [batch, seq]),
    ``types`` the matching pseudo-token types (-1 text), ``tokens`` [T, L] the
    aligned image tokens in image order, ``sentinels`` [3, L] the image_start,
    image_newline and image_end embeddings.  Reading "merge_embeddings".
    """
    out = np.array(embeds, copy=True)
    flat = out.reshape(-1, out.shape[-1])
    kinds = np.asarray(types).reshape(-1)
    sentinel_row = {NL_START: 0, NL_NEWLINE: 1, NL_END: 2}
    t = 0
    for pos in range(len(kinds)):
        kind = int(kinds[pos])
        if kind == NL_IMAGE:
            flat[pos] = tokens[t]
            t += 1
        elif kind in sentinel_row:
            flat[pos] = sentinels[sentinel_row[kind]]
    return out


def encode(patches, gh, gw, weights, n_heads, eps=1e-6, theta=10000.0, with_aligner=True,
           dtype=np.float64, pad_odd=False):
    """[MOD] DeepseekV4Model.encode_image: the vision tower, then the aligner."""
    x = tower(patches, gh, gw, weights, n_heads, eps, theta, dtype)
    if not with_aligner:
        return x
    return aligner(x, gh, gw, weights["aligner"], dtype=dtype, pad_odd=pad_odd)


def encode_varlen(patches, grids, weights, n_heads, eps=1e-6, theta=10000.0, with_aligner=True,
                  dtype=np.float64, pad_odd=False):
    """Concatenated images ([MOD] pixel_values + image_grid_hws): each image alone, in order."""
    outs = []
    off = 0
    for gh, gw in grids:
        P = gh * gw
        outs.append(encode(patches[off:off + P], gh, gw, weights, n_heads, eps, theta,
                           with_aligner, dtype, pad_odd))
        off += P
    return np.concatenate(outs, axis=0)
