"""ctypes view of ``libvitenc.so`` (declarations mirror ``include/vitenc.h``).

Loading fails loudly when the library has not been built: there is no fallback
path, every step of the encoder runs in the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvitenc.so")

VIT_OK, VIT_E_ARG, VIT_E_SHAPE, VIT_E_ODD_GRID, VIT_E_WORKSPACE, VIT_E_HIP = 0, -1, -2, -3, -4, -5
VIT_BF16, VIT_F32 = 0, 1
VIT_NO_ALIGNER, VIT_OUT_NLAYOUT, VIT_IN_PIXELS, VIT_ALIGN_PAD = 1, 2, 4, 8
VIT_MAX_IMAGES = 128
VIT_EPI_STORE, VIT_EPI_STORE_F32, VIT_EPI_ADD_F32, VIT_EPI_SWIGLU = 0, 1, 2, 3
VIT_EPI_BIAS, VIT_EPI_BIAS_GELU = 4, 5
KERNEL_CLASSES = ["embed", "rmsnorm", "qkv", "rope", "attn", "outproj", "gateup", "down",
                  "gather", "aligner", "merge", "lngather", "proj1", "proj2", "bwd_gemm",
                  "bwd_dn", "bwd_pass", "bwd_attn"]

c_i32, c_i64, c_f32, c_vp, c_size = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_size_t)
P_i32 = ctypes.POINTER(ctypes.c_int32)


class VitConfig(ctypes.Structure):
    _fields_ = [("vision_dim", c_i32), ("n_heads", c_i32), ("head_dim", c_i32),
                ("mlp_hidden", c_i32), ("n_blocks", c_i32), ("patch_dim", c_i32),
                ("merge", c_i32), ("llm_dim", c_i32), ("rope_theta", c_f32),
                ("rms_eps", c_f32), ("dtype", c_i32)]


class VitWeights(ctypes.Structure):
    _fields_ = [("patch_embed", c_vp), ("wqkv", ctypes.POINTER(c_vp)),
                ("wo", ctypes.POINTER(c_vp)), ("w_gate", ctypes.POINTER(c_vp)),
                ("w_up", ctypes.POINTER(c_vp)), ("w_down", ctypes.POINTER(c_vp)),
                ("norm1", ctypes.POINTER(c_vp)), ("norm2", ctypes.POINTER(c_vp)),
                ("final_norm", c_vp), ("aligner", c_vp)]


class VitMerger(ctypes.Structure):
    _fields_ = [("dim", c_i32), ("hidden", c_i32), ("out_dim", c_i32), ("eps", c_f32),
                ("ln_w", c_vp), ("ln_b", c_vp), ("w1", c_vp), ("b1", c_vp), ("w2", c_vp),
                ("b2", c_vp)]


class VitMlpGrad(ctypes.Structure):
    _fields_ = [("rows", c_i64), ("dim", c_i32), ("hidden", c_i32), ("eps", c_f32),
                ("x", c_vp), ("norm_w", c_vp), ("w_gate", c_vp), ("w_up", c_vp), ("w_down", c_vp),
                ("dy", c_vp), ("dx", c_vp), ("d_norm_w", c_vp), ("d_w_gate", c_vp),
                ("d_w_up", c_vp), ("d_w_down", c_vp)]


class VitTowerGrads(ctypes.Structure):
    _fields_ = [("d_patch_embed", c_vp), ("d_wqkv", ctypes.POINTER(c_vp)),
                ("d_wo", ctypes.POINTER(c_vp)), ("d_w_gate", ctypes.POINTER(c_vp)),
                ("d_w_up", ctypes.POINTER(c_vp)), ("d_w_down", ctypes.POINTER(c_vp)),
                ("d_norm1", ctypes.POINTER(c_vp)), ("d_norm2", ctypes.POINTER(c_vp)),
                ("d_final_norm", c_vp)]


class VitAttnGrad(ctypes.Structure):
    _fields_ = [("dim", c_i32), ("n_heads", c_i32), ("rope_theta", c_f32), ("eps", c_f32),
                ("x", c_vp), ("norm_w", c_vp), ("wqkv", c_vp), ("wo", c_vp), ("dy", c_vp),
                ("dx", c_vp), ("d_norm_w", c_vp), ("d_wqkv", c_vp), ("d_wo", c_vp)]


# name -> (restype, argtypes); every function declared in include/vitenc.h
SIGNATURES = {
    "vit_status_str": (ctypes.c_char_p, [c_i32]),
    "vit_last_error": (ctypes.c_char_p, []),
    "vit_workspace_bytes": (c_size, [ctypes.POINTER(VitConfig), P_i32, c_i32, c_i32]),
    "vit_encode": (c_i32, [ctypes.POINTER(VitConfig), ctypes.POINTER(VitWeights), c_vp, c_i32,
                           c_i32, c_i32, c_vp, c_vp, c_size, c_vp]),
    "vit_encode_varlen": (c_i32, [ctypes.POINTER(VitConfig), ctypes.POINTER(VitWeights), c_vp,
                                  P_i32, c_i32, c_i32, c_vp, c_vp, c_size, c_vp]),
    "vit_encode_varlen_noalloc": (c_i32, [ctypes.POINTER(VitConfig), ctypes.POINTER(VitWeights),
                                          c_vp, P_i32, c_i32, c_i32, c_vp, c_vp]),
    "vit_noalloc_workspace_limit": (c_size, []),
    "vit_aligner_layout": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "vit_rmsnorm": (c_i32, [c_vp, c_vp, c_f32, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "vit_rope_table": (c_i32, [P_i32, c_i32, c_i32, c_f32, c_vp, c_vp]),
    "vit_rope": (c_i32, [c_i32, c_vp, c_vp, c_i64, c_i32, c_i32, c_vp]),
    "vit_attention_workspace_bytes": (c_size, [c_i32, P_i32, c_i32, c_i32, c_i32]),
    "vit_attention_varlen": (c_i32, [c_i32, c_vp, P_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_size,
                                     c_vp]),
    "vit_gemm": (c_i32, [c_i32, c_i32, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64,
                         c_i64, c_vp]),
    "vit_aligner_gather": (c_i32, [c_i32, c_vp, P_i32, c_i32, c_i32, c_vp, c_vp]),
    "vit_patch_merger_workspace_bytes": (c_size, [ctypes.POINTER(VitMerger), P_i32, c_i32]),
    "vit_patch_merger": (c_i32, [ctypes.POINTER(VitMerger), c_vp, P_i32, c_i32, c_vp, c_vp, c_size,
                                 c_vp]),
    "vit_layernorm_gather": (c_i32, [c_vp, P_i32, c_i32, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp]),
    "vit_gemm_bias": (c_i32, [c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64,
                              c_i64, c_vp]),
    "vit_attn_backward_workspace_bytes": (c_size, [ctypes.POINTER(VitAttnGrad), P_i32, c_i32]),
    "vit_attn_backward": (c_i32, [ctypes.POINTER(VitAttnGrad), P_i32, c_i32, c_vp, c_size, c_vp]),
    "vit_tower_backward_workspace_bytes": (c_size, [ctypes.POINTER(VitConfig), P_i32, c_i32]),
    "vit_tower_backward": (c_i32, [ctypes.POINTER(VitConfig), ctypes.POINTER(VitWeights), c_vp,
                                   P_i32, c_i32, c_vp, ctypes.POINTER(VitTowerGrads), c_vp,
                                   c_size, c_vp]),
    "vit_mlp_backward_workspace_bytes": (c_size, [c_i64, c_i32, c_i32]),
    "vit_mlp_backward": (c_i32, [ctypes.POINTER(VitMlpGrad), c_vp, c_size, c_vp]),
    "vit_mfma_peak_out_floats": (c_i64, []),
    "vit_mfma_peak": (c_i32, [c_i32, c_vp, ctypes.POINTER(ctypes.c_double), c_vp]),
    "vit_merge_workspace_bytes": (c_size, [c_i64]),
    "vit_merge_image_embeddings": (c_i32, [c_i32, c_vp, c_i64, c_i32, c_vp, c_vp, c_i64, c_vp,
                                           c_vp, c_vp, c_size, c_vp]),
    "vit_profile_enable": (c_i32, [c_i32, c_i32]),
    "vit_profile_read": (c_i32, [c_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
}

_lock = threading.Lock()
_lib = None


class VitError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


def load() -> ctypes.CDLL:
    """Load the built HIP library (raises if it is missing: no CPU fallback exists)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -c 'import __graft_entry__ as g; g.build()')")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def check(status: int, where: str) -> None:
    if status != VIT_OK:
        lib = load()
        detail = lib.vit_last_error().decode() or lib.vit_status_str(status).decode()
        raise VitError(status, where, detail)


def grid_array(grids):
    flat = [int(v) for g in grids for v in g]
    return (ctypes.c_int32 * len(flat))(*flat)
