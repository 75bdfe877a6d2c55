"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module draws random numbers and rounds them to the storage precision;
it holds none of the encoder's arithmetic.  Both sides receive the same
arrays from here.

Recipe (one numpy ``Generator(PCG64(seed))`` per workload, fixed order):
  1. patches ``[P, 588]`` uniform on [-1, 1)          (normalised RGB patches)
  2. patch-embed weight ``[d, 588]`` N(0, 0.02)
  3. per block: norm1 ``[d]`` 1+N(0,0.02); wqkv ``[3d, d]``; wo ``[d, d]``;
     norm2 ``[d]``; w_gate ``[h, d]``; w_up ``[h, d]``; w_down ``[d, h]``
  4. final norm ``[d]`` 1+N(0, 0.02)
  5. aligner weight ``[L, 4d]`` N(0, 0.02) (only when the workload has one)
In bf16 workloads the patches and every matrix are rounded to bfloat16
(round-to-nearest-even) and kept as float32 arrays holding bf16 values; norm
scales stay float32 (the vision RMSNorm keeps an fp32 scale parameter).
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

INIT_STD = 0.02


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def make_inputs(cfg, seed: int) -> Dict:
    """Return {"patches", "grids", "weights"} for one workload (see module doc)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bf16 = cfg.dtype == "bf16"
    P, K, d, h = cfg.total_patches, cfg.patch_dim, cfg.vision_dim, cfg.mlp_hidden

    def mat(rows, cols):
        m = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(INIT_STD)
        return round_to_bf16(m) if bf16 else m

    def scale(n):
        return (np.float32(1.0) + rng.standard_normal(n, dtype=np.float32) * np.float32(INIT_STD))

    patches = rng.random((P, K), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if bf16:
        patches = round_to_bf16(patches)
    w = {"patch_embed": mat(d, K), "blocks": []}
    for _ in range(cfg.n_blocks):
        blk = {}
        blk["norm1"] = scale(d)
        blk["wqkv"] = mat(3 * d, d)
        blk["wo"] = mat(d, d)
        blk["norm2"] = scale(d)
        blk["w_gate"] = mat(h, d)
        blk["w_up"] = mat(h, d)
        blk["w_down"] = mat(d, h)
        w["blocks"].append(blk)
    w["final_norm"] = scale(d)
    w["aligner"] = mat(cfg.llm_dim, cfg.merge * cfg.merge * d) if cfg.aligner else None
    return {"patches": patches, "grids": [tuple(g) for g in cfg.grids], "weights": w}


def random_array(shape, seed: int, kind: str = "normal", std: float = 1.0,
                 bf16: bool = False) -> np.ndarray:
    """A seeded float32 array for per-step tests ("normal" or "uniform" on [-1,1))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    elif kind == "uniform":
        a = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(kind)
    return round_to_bf16(a) if bf16 else a


def make_merger_weights(dim: int, hidden: int, out_dim: int, seed: int) -> Dict:
    """Seeded PatchMerger projector weights: norm weight 1 + N(0, 0.02) and bias
    N(0, 0.02) (float32), matrices N(0, 0.02) rounded to bf16 ([out, in]), biases
    N(0, 0.02) (float32)."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def normal(*shape):
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)

    return {"ln_w": np.float32(1.0) + normal(dim), "ln_b": normal(dim),
            "w1": round_to_bf16(normal(hidden, 4 * dim)), "b1": normal(hidden),
            "w2": round_to_bf16(normal(out_dim, hidden)), "b2": normal(out_dim)}


def seqlens(grids: List) -> List[int]:
    return [int(gh) * int(gw) for gh, gw in grids]
