"""Python binding of the gfx950 encoder library (argument marshalling only).

PyTorch provides device memory and the current HIP stream; every step of the
encoder runs inside ``libvitenc.so``.  Names follow the C ABI in
``include/vitenc.h``.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib
from .configs import VitConfig

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_CODE = {"bf16": _lib.VIT_BF16, "f32": _lib.VIT_F32}


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors passed to the HIP library must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to the HIP library must be contiguous")


def c_config(cfg: VitConfig) -> _lib.VitConfig:
    return _lib.VitConfig(cfg.vision_dim, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden, cfg.n_blocks,
                          cfg.patch_dim, cfg.merge, cfg.llm_dim, cfg.rope_theta, cfg.rms_eps,
                          _CODE[cfg.dtype])


class DeviceWeights:
    """Encoder weights resident on the GPU plus the C struct pointing at them."""

    def __init__(self, cfg: VitConfig, host: Dict, device="cuda"):
        dt = _TORCH_DTYPE[cfg.dtype]

        def mat(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dt)

        def vec(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device)

        self.cfg = cfg
        self.patch_embed = mat(host["patch_embed"])
        self.blocks = []
        for b in host["blocks"]:
            self.blocks.append({k: (vec(v) if k.startswith("norm") else mat(v)) for k, v in b.items()})
        self.final_norm = vec(host["final_norm"])
        self.aligner = mat(host["aligner"]) if host.get("aligner") is not None else None
        n = len(self.blocks)

        def arr(key):
            return (ctypes.c_void_p * max(n, 1))(*[b[key].data_ptr() for b in self.blocks])

        self._arrays = {k: arr(k) for k in ("wqkv", "wo", "w_gate", "w_up", "w_down", "norm1", "norm2")}
        self.c = _lib.VitWeights(
            self.patch_embed.data_ptr(), self._arrays["wqkv"], self._arrays["wo"],
            self._arrays["w_gate"], self._arrays["w_up"], self._arrays["w_down"],
            self._arrays["norm1"], self._arrays["norm2"], self.final_norm.data_ptr(),
            None if self.aligner is None else self.aligner.data_ptr())


def output_rows(cfg: VitConfig, grids: Sequence[Tuple[int, int]], aligner: bool, nlayout: bool,
                pad_odd: bool = False) -> int:
    """Rows of the encoder output (merged grids rounded up with pad_odd)."""
    if not aligner:
        return sum(h * w for h, w in grids)
    m = cfg.merge

    def q(v):
        return -(-v // m) if pad_odd else v // m

    if nlayout:
        return sum(q(h) * (q(w) + 1) + 2 for h, w in grids)
    return sum(q(h) * q(w) for h, w in grids)


def _flags(aligner: bool, nlayout: bool, pixels: bool, pad_odd: bool = False) -> int:
    return ((0 if aligner else _lib.VIT_NO_ALIGNER) | (_lib.VIT_OUT_NLAYOUT if nlayout else 0)
            | (_lib.VIT_IN_PIXELS if pixels else 0) | (_lib.VIT_ALIGN_PAD if pad_odd else 0))


def workspace_bytes(cfg: VitConfig, grids, aligner=True, nlayout=False, pixels=False,
                    pad_odd=False) -> int:
    lib = _lib.load()
    flags = _flags(aligner, nlayout, pixels, pad_odd)
    c = c_config(cfg)
    n = lib.vit_workspace_bytes(ctypes.byref(c), _lib.grid_array(grids), len(grids), flags)
    if n == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_workspace_bytes")
    return n


class Encoder:
    """Reusable encoder call: keeps the workspace for one set of grids."""

    def __init__(self, cfg: VitConfig, weights: DeviceWeights, grids, aligner=True, nlayout=False,
                 device="cuda", pixels=False, pad_odd=False):
        self.cfg, self.w = cfg, weights
        self.grids = [tuple(int(v) for v in g) for g in grids]
        self.aligner, self.nlayout = aligner, nlayout
        self.flags = _flags(aligner, nlayout, pixels, pad_odd)
        self.ws_bytes = workspace_bytes(cfg, self.grids, aligner, nlayout, pixels, pad_odd)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.c_cfg = c_config(cfg)
        self.c_grids = _lib.grid_array(self.grids)
        cols = cfg.llm_dim if aligner else cfg.vision_dim
        self.out_shape = (output_rows(cfg, self.grids, aligner, nlayout, pad_odd), cols)
        self.device = device

    def __call__(self, patches: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        _require_cuda(patches)
        if out is None:
            alloc = torch.zeros if self.nlayout else torch.empty
            out = alloc(self.out_shape, dtype=_TORCH_DTYPE[self.cfg.dtype], device=self.device)
        _require_cuda(out)
        lib = _lib.load()
        st = lib.vit_encode_varlen(ctypes.byref(self.c_cfg), ctypes.byref(self.w.c),
                                   patches.data_ptr(), self.c_grids, len(self.grids), self.flags,
                                   out.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                                   _stream(patches.device))
        _lib.check(st, "vit_encode_varlen")
        return out


def encode(patches: torch.Tensor, grid: Tuple[int, int], weights: DeviceWeights, aligner=True,
           nlayout=False, pixels=False, pad_odd=False) -> torch.Tensor:
    """vit_encode: one image [gh*gw, patch_dim] (or with pixels=True the pixel image
    [3, ps*gh, ps*gw]) -> aligned tokens (or encoded patches)."""
    cfg = weights.cfg
    _require_cuda(patches)
    ws_bytes = workspace_bytes(cfg, [grid], aligner, nlayout, pixels, pad_odd)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=patches.device)
    cols = cfg.llm_dim if aligner else cfg.vision_dim
    rows = output_rows(cfg, [grid], aligner, nlayout, pad_odd)
    out = (torch.zeros if nlayout else torch.empty)((rows, cols), dtype=_TORCH_DTYPE[cfg.dtype],
                                                     device=patches.device)
    flags = _flags(aligner, nlayout, pixels, pad_odd)
    c = c_config(cfg)
    lib = _lib.load()
    st = lib.vit_encode(ctypes.byref(c), ctypes.byref(weights.c), patches.data_ptr(), grid[0],
                        grid[1], flags, out.data_ptr(), ws.data_ptr(), ws_bytes,
                        _stream(patches.device))
    _lib.check(st, "vit_encode")
    return out


def encode_varlen(patches: torch.Tensor, grids, weights: DeviceWeights, aligner=True,
                  nlayout=False, pixels=False, pad_odd=False) -> torch.Tensor:
    """vit_encode_varlen: packed images with block-diagonal attention (patches, or
    with pixels=True the pixel images back to back; pad_odd zero-pads odd grids
    for the 2x2 merge)."""
    return Encoder(weights.cfg, weights, grids, aligner, nlayout, patches.device, pixels,
                   pad_odd)(patches)


def aligner_layout(grid_h: int, grid_w: int, merge: int = 2, device="cuda"):
    """vit_aligner_layout -> (perm, nl_type, nl_src) int32 tensors."""
    P = grid_h * grid_w
    L = (grid_h // merge) * (grid_w // merge + 1) + 2
    perm = torch.empty(P, dtype=torch.int32, device=device)
    nl_type = torch.empty(L, dtype=torch.int32, device=device)
    nl_src = torch.empty(L, dtype=torch.int32, device=device)
    st = _lib.load().vit_aligner_layout(grid_h, grid_w, merge, perm.data_ptr(), nl_type.data_ptr(),
                                        nl_src.data_ptr(), _stream(device))
    _lib.check(st, "vit_aligner_layout")
    return perm, nl_type, nl_src


# ---------------------------------------------------------------- step entry points
def rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out_dtype="bf16") -> torch.Tensor:
    _require_cuda(x, w)
    assert x.dtype == torch.float32 and w.dtype == torch.float32
    out = torch.empty(x.shape, dtype=_TORCH_DTYPE[out_dtype], device=x.device)
    st = _lib.load().vit_rmsnorm(x.data_ptr(), w.data_ptr(), eps, x.shape[0], x.shape[1],
                                 _CODE[out_dtype], out.data_ptr(), _stream(x.device))
    _lib.check(st, "vit_rmsnorm")
    return out


def rope_table(grids, head_dim: int, theta: float = 10000.0, device="cuda") -> torch.Tensor:
    P = sum(h * w for h, w in grids)
    table = torch.empty((P, head_dim // 2, 2), dtype=torch.float32, device=device)
    st = _lib.load().vit_rope_table(_lib.grid_array(grids), len(grids), head_dim, theta,
                                    table.data_ptr(), _stream(device))
    _lib.check(st, "vit_rope_table")
    return table


def rope_(qkv: torch.Tensor, table: torch.Tensor, n_heads: int, head_dim: int) -> torch.Tensor:
    _require_cuda(qkv, table)
    code = _lib.VIT_BF16 if qkv.dtype == torch.bfloat16 else _lib.VIT_F32
    st = _lib.load().vit_rope(code, qkv.data_ptr(), table.data_ptr(), qkv.shape[0], n_heads,
                              head_dim, _stream(qkv.device))
    _lib.check(st, "vit_rope")
    return qkv


def attention_varlen(qkv: torch.Tensor, grids, n_heads: int, head_dim: int) -> torch.Tensor:
    _require_cuda(qkv)
    code = _lib.VIT_BF16 if qkv.dtype == torch.bfloat16 else _lib.VIT_F32
    out = torch.empty((qkv.shape[0], n_heads * head_dim), dtype=qkv.dtype, device=qkv.device)
    lib = _lib.load()
    g = _lib.grid_array(grids)
    nbytes = lib.vit_attention_workspace_bytes(code, g, len(grids), n_heads, head_dim)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=qkv.device)
    st = lib.vit_attention_varlen(code, qkv.data_ptr(), g, len(grids), n_heads, head_dim,
                                  out.data_ptr(), ws.data_ptr(), nbytes, _stream(qkv.device))
    _lib.check(st, "vit_attention_varlen")
    return out


def gemm(A: torch.Tensor, B: torch.Tensor, epilogue: int = _lib.VIT_EPI_STORE,
         B2: Optional[torch.Tensor] = None, C: Optional[torch.Tensor] = None) -> torch.Tensor:
    """vit_gemm: C = epilogue(A . B^T) (A [M, K], B/B2 [N, K])."""
    _require_cuda(A, B, B2, C)
    code = _lib.VIT_BF16 if A.dtype == torch.bfloat16 else _lib.VIT_F32
    M, K = A.shape
    N = B.shape[0]
    if C is None:
        odt = torch.float32 if epilogue in (_lib.VIT_EPI_STORE_F32, _lib.VIT_EPI_ADD_F32) else A.dtype
        C = torch.zeros((M, N), dtype=odt, device=A.device)
    st = _lib.load().vit_gemm(code, epilogue, A.data_ptr(), A.stride(0), B.data_ptr(), _ptr(B2),
                              B.stride(0), C.data_ptr(), C.stride(0), M, N, K, _stream(A.device))
    _lib.check(st, "vit_gemm")
    return C


def aligner_gather(x: torch.Tensor, grids, merge: int = 2) -> torch.Tensor:
    _require_cuda(x)
    code = _lib.VIT_BF16 if x.dtype == torch.bfloat16 else _lib.VIT_F32
    T = sum(h * w for h, w in grids) // (merge * merge)
    G = torch.empty((T, merge * merge * x.shape[1]), dtype=x.dtype, device=x.device)
    st = _lib.load().vit_aligner_gather(code, x.data_ptr(), _lib.grid_array(grids), len(grids),
                                        x.shape[1], G.data_ptr(), _stream(x.device))
    _lib.check(st, "vit_aligner_gather")
    return G


class MergerWeights:
    """PatchMerger projector weights on the device: norm weight / bias, two biased
    linear maps (bf16 matrices ``[out, in]``, float32 vectors)."""

    def __init__(self, host: Dict, eps: float = 1e-6, device="cuda"):
        def mat(a):
            return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(device, torch.bfloat16).contiguous()

        def vec(a):
            return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(device).contiguous()

        self.ln_w, self.ln_b = vec(host["ln_w"]), vec(host["ln_b"])
        self.w1, self.b1 = mat(host["w1"]), vec(host["b1"])
        self.w2, self.b2 = mat(host["w2"]), vec(host["b2"])
        self.dim = self.ln_w.numel()
        self.hidden, self.out_dim = self.w1.shape[0], self.w2.shape[0]
        self.c = _lib.VitMerger(self.dim, self.hidden, self.out_dim, eps, self.ln_w.data_ptr(),
                                self.ln_b.data_ptr(), self.w1.data_ptr(), self.b1.data_ptr(),
                                self.w2.data_ptr(), self.b2.data_ptr())


def merger_workspace_bytes(mw: MergerWeights, grids) -> int:
    n = _lib.load().vit_patch_merger_workspace_bytes(ctypes.byref(mw.c), _lib.grid_array(grids),
                                                      len(grids))
    if n == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_patch_merger_workspace_bytes")
    return n


def patch_merger(x: torch.Tensor, grids, mw: MergerWeights, out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """vit_patch_merger: x [sum P, dim] bf16 (the encoder output) -> [sum P/4, out_dim]."""
    _require_cuda(x, out, ws)
    lib = _lib.load()
    g = _lib.grid_array(grids)
    need = lib.vit_patch_merger_workspace_bytes(ctypes.byref(mw.c), g, len(grids))
    if need == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_patch_merger_workspace_bytes")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    T = sum(h * w for h, w in grids) // 4
    if out is None:
        out = torch.empty((T, mw.out_dim), dtype=torch.bfloat16, device=x.device)
    st = lib.vit_patch_merger(ctypes.byref(mw.c), x.data_ptr(), g, len(grids), out.data_ptr(),
                              ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(st, "vit_patch_merger")
    return out


def layernorm_gather(x: torch.Tensor, grids, ln_w: torch.Tensor, ln_b: torch.Tensor,
                     eps: float = 1e-6) -> torch.Tensor:
    """vit_layernorm_gather: G [sum P/4, 4*dim] bf16."""
    _require_cuda(x, ln_w, ln_b)
    T = sum(h * w for h, w in grids) // 4
    G = torch.empty((T, 4 * x.shape[1]), dtype=torch.bfloat16, device=x.device)
    st = _lib.load().vit_layernorm_gather(x.data_ptr(), _lib.grid_array(grids), len(grids),
                                          x.shape[1], ln_w.data_ptr(), ln_b.data_ptr(), eps,
                                          G.data_ptr(), _stream(x.device))
    _lib.check(st, "vit_layernorm_gather")
    return G


def gemm_bias(A: torch.Tensor, B: torch.Tensor, bias: torch.Tensor, gelu: bool = False) -> torch.Tensor:
    """vit_gemm_bias: C = A . B^T + bias, or gelu of it (bf16 in and out, fp32 bias)."""
    _require_cuda(A, B, bias)
    M, K = A.shape
    N = B.shape[0]
    C = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    epi = _lib.VIT_EPI_BIAS_GELU if gelu else _lib.VIT_EPI_BIAS
    st = _lib.load().vit_gemm_bias(epi, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0),
                                   bias.data_ptr(), C.data_ptr(), C.stride(0), M, N, K,
                                   _stream(A.device))
    _lib.check(st, "vit_gemm_bias")
    return C


def mlp_backward(x: torch.Tensor, norm_w: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                 w_down: torch.Tensor, dy: torch.Tensor, eps: float = 1e-6,
                 ws: Optional[torch.Tensor] = None):
    """vit_mlp_backward: gradients of y = x + mlp(norm2(x)) for dy; returns
    (dx, d_norm_w, d_w_gate, d_w_up, d_w_down), all float32."""
    _require_cuda(x, norm_w, w_gate, w_up, w_down, dy, ws)
    P, d = x.shape
    h = w_gate.shape[0]
    lib = _lib.load()
    need = lib.vit_mlp_backward_workspace_bytes(P, d, h)
    if need == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_mlp_backward_workspace_bytes")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    dx, dnw = torch.empty((P, d), **f32), torch.empty(d, **f32)
    dwg, dwu, dwd = torch.empty((h, d), **f32), torch.empty((h, d), **f32), torch.empty((d, h), **f32)
    args = _lib.VitMlpGrad(P, d, h, eps, x.data_ptr(), norm_w.data_ptr(), w_gate.data_ptr(),
                           w_up.data_ptr(), w_down.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                           dnw.data_ptr(), dwg.data_ptr(), dwu.data_ptr(), dwd.data_ptr())
    st = lib.vit_mlp_backward(ctypes.byref(args), ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(st, "vit_mlp_backward")
    return dx, dnw, dwg, dwu, dwd


def attn_backward(x: torch.Tensor, norm_w: torch.Tensor, wqkv: torch.Tensor, wo: torch.Tensor,
                  dy: torch.Tensor, grids, n_heads: int, theta: float = 10000.0,
                  eps: float = 1e-6, ws: Optional[torch.Tensor] = None):
    """vit_attn_backward: gradients of y = x + attn(norm1(x)) for dy over packed
    images; returns (dx, d_norm_w, d_wqkv, d_wo), all float32."""
    _require_cuda(x, norm_w, wqkv, wo, dy, ws)
    P, d = x.shape
    f32 = dict(dtype=torch.float32, device=x.device)
    dx, dnw = torch.empty((P, d), **f32), torch.empty(d, **f32)
    dwqkv, dwo = torch.empty((3 * d, d), **f32), torch.empty((d, d), **f32)
    args = _lib.VitAttnGrad(d, n_heads, theta, eps, x.data_ptr(), norm_w.data_ptr(),
                            wqkv.data_ptr(), wo.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                            dnw.data_ptr(), dwqkv.data_ptr(), dwo.data_ptr())
    lib = _lib.load()
    g = _lib.grid_array(grids)
    need = lib.vit_attn_backward_workspace_bytes(ctypes.byref(args), g, len(grids))
    if need == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_attn_backward_workspace_bytes")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = lib.vit_attn_backward(ctypes.byref(args), g, len(grids), ws.data_ptr(), ws.numel(),
                               _stream(x.device))
    _lib.check(st, "vit_attn_backward")
    return dx, dnw, dwqkv, dwo


TOWER_GRAD_KEYS = ("norm1", "wqkv", "wo", "norm2", "w_gate", "w_up", "w_down")


def tower_backward_workspace_bytes(cfg: VitConfig, grids) -> int:
    c = c_config(cfg)
    n = _lib.load().vit_tower_backward_workspace_bytes(ctypes.byref(c), _lib.grid_array(grids),
                                                        len(grids))
    if n == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_tower_backward_workspace_bytes")
    return n


def tower_backward(patches: torch.Tensor, grids, w: "DeviceWeights", dy: torch.Tensor,
                   ws: Optional[torch.Tensor] = None) -> Dict:
    """vit_tower_backward: gradients of every tower weight for dy = dL/d(output of
    the final norm) over packed images (patches [sum P, patch_dim] bf16, dy float32
    [sum P, vision_dim]).  Returns float32 tensors in a dict shaped like the
    weights: ``patch_embed``, ``final_norm`` and ``blocks`` (one dict per block)."""
    _require_cuda(patches, dy, ws)
    cfg = w.cfg
    d, h, pd = cfg.vision_dim, cfg.mlp_hidden, cfg.patch_dim
    f32 = dict(dtype=torch.float32, device=patches.device)
    shapes = {"norm1": (d,), "wqkv": (3 * d, d), "wo": (d, d), "norm2": (d,), "w_gate": (h, d),
              "w_up": (h, d), "w_down": (d, h)}
    out = {"patch_embed": torch.empty((d, pd), **f32), "final_norm": torch.empty(d, **f32),
           "blocks": [{k: torch.empty(shapes[k], **f32) for k in TOWER_GRAD_KEYS}
                      for _ in range(cfg.n_blocks)]}
    n = cfg.n_blocks

    def arr(key):
        return (ctypes.c_void_p * max(n, 1))(*[b[key].data_ptr() for b in out["blocks"]])

    arrays = {k: arr(k) for k in TOWER_GRAD_KEYS}
    grads = _lib.VitTowerGrads(out["patch_embed"].data_ptr(), arrays["wqkv"], arrays["wo"],
                               arrays["w_gate"], arrays["w_up"], arrays["w_down"], arrays["norm1"],
                               arrays["norm2"], out["final_norm"].data_ptr())
    c = c_config(cfg)
    lib = _lib.load()
    g = _lib.grid_array(grids)
    if ws is None:
        ws = torch.empty(tower_backward_workspace_bytes(cfg, grids), dtype=torch.uint8,
                         device=patches.device)
    st = lib.vit_tower_backward(ctypes.byref(c), ctypes.byref(w.c), patches.data_ptr(), g,
                                len(grids), dy.data_ptr(), ctypes.byref(grads), ws.data_ptr(),
                                ws.numel(), _stream(patches.device))
    _lib.check(st, "vit_tower_backward")
    return out


def mfma_peak_tflops(iters: int = 20000, reps: int = 5, device="cuda") -> float:
    """vit_mfma_peak: the best of `reps` timed calls of the dense-MFMA probe, in
    TFLOP/s (bf16)."""
    lib = _lib.load()
    out = torch.empty(lib.vit_mfma_peak_out_floats(), dtype=torch.float32, device=device)
    flops = ctypes.c_double()
    st = _stream(out.device)
    _lib.check(lib.vit_mfma_peak(iters, out.data_ptr(), ctypes.byref(flops), st), "vit_mfma_peak")
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _lib.check(lib.vit_mfma_peak(iters, out.data_ptr(), ctypes.byref(flops), st),
                   "vit_mfma_peak")
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def merge_workspace_bytes(positions: int) -> int:
    n = _lib.load().vit_merge_workspace_bytes(int(positions))
    if n == 0:
        _lib.check(_lib.VIT_E_SHAPE, "vit_merge_workspace_bytes")
    return n


def merge_image_embeddings_(embeds: torch.Tensor, types: torch.Tensor, tokens: torch.Tensor,
                            sentinels: torch.Tensor, ws: Optional[torch.Tensor] = None,
                            n_image: Optional[torch.Tensor] = None) -> torch.Tensor:
    """vit_merge_image_embeddings, in place on ``embeds`` [..., hidden].

    ``types`` (int32, one code per row of embeds: 0 START, 1 IMAGE, 2 NEWLINE,
    3 END, other text), ``tokens`` [n_tokens, hidden], ``sentinels`` [3, hidden]
    (start, newline, end).  ``n_image`` (int32 [1], optional) receives the number
    of IMAGE positions.
    """
    _require_cuda(embeds, types, tokens, sentinels, ws, n_image)
    if types.dtype != torch.int32 or (n_image is not None and n_image.dtype != torch.int32):
        raise ValueError("types and n_image must be int32")
    if not (embeds.dtype == tokens.dtype == sentinels.dtype):
        raise ValueError("embeds, tokens and sentinels must share one dtype")
    hidden = embeds.shape[-1]
    positions = embeds.numel() // hidden if hidden else 0
    if types.numel() != positions or tokens.shape[-1] != hidden or tuple(sentinels.shape) != (3, hidden):
        raise ValueError("shape mismatch between embeds, types, tokens and sentinels")
    code = _lib.VIT_BF16 if embeds.dtype == torch.bfloat16 else _lib.VIT_F32
    need = merge_workspace_bytes(positions)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=embeds.device)
    st = _lib.load().vit_merge_image_embeddings(
        code, embeds.data_ptr(), positions, hidden, types.data_ptr(), tokens.data_ptr(),
        tokens.shape[0], sentinels.data_ptr(), _ptr(n_image), ws.data_ptr(), ws.numel(),
        _stream(embeds.device))
    _lib.check(st, "vit_merge_image_embeddings")
    return embeds


def profile_enable(kernel: str, on: bool = True) -> None:
    _lib.check(_lib.load().vit_profile_enable(_lib.KERNEL_CLASSES.index(kernel), int(on)),
               "vit_profile_enable")


def profile_read(kernel: str) -> Tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _lib.check(_lib.load().vit_profile_read(_lib.KERNEL_CLASSES.index(kernel), ctypes.byref(ms),
                                            ctypes.byref(n)), "vit_profile_read")
    return ms.value, n.value
