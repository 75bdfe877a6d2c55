"""Named encoder workloads (dimensions only; no arithmetic of the method).

The encoder shape follows the DeepSeek-V4-Flash-Vision vision module page
(classes DeepseekV4VisionTransformer / Block / Attention / MLP / Aligner):
``head_dim = vision_dim // n_heads``, RMSNorm eps 1e-6, a 2x2 aligner merge.
The concrete sizes (vision_dim, heads, MLP hidden, block count, LLM width) are
not printed on the pages; the five workloads below fix them.  The ragged grids
27x37, 37x27, 10x78, 112x7 and the square 28x28 are the ViT grids of the
NeMo Automodel PR #3772 "Validation > vision-only parity" table.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

PATCH_SIZE = 14
PATCH_DIM = 3 * PATCH_SIZE * PATCH_SIZE  # 588 flattened RGB values per patch


@dataclasses.dataclass(frozen=True)
class VitConfig:
    name: str
    grids: Tuple[Tuple[int, int], ...]  # (rows, cols) per image
    vision_dim: int
    n_heads: int
    mlp_hidden: int
    n_blocks: int
    llm_dim: int  # 0 = encoder only, no aligner
    dtype: str  # "bf16" or "f32"
    patch_size: int = PATCH_SIZE
    merge: int = 2
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.vision_dim // self.n_heads

    @property
    def patch_dim(self) -> int:
        return 3 * self.patch_size * self.patch_size

    @property
    def aligner(self) -> bool:
        return self.llm_dim > 0

    @property
    def total_patches(self) -> int:
        return sum(h * w for h, w in self.grids)

    @property
    def seqlens(self) -> List[int]:
        return [h * w for h, w in self.grids]

    def block_flops(self) -> float:
        """Algorithmic FLOPs of one encoder block over the whole batch.

        QKV 6Pd^2 + out-proj 2Pd^2 + gate/up 4Pdh + down 2Pdh + QK^T and PV
        4 d P_i^2 per image.  Softmax and norms are not counted.
        """
        P, d, h = self.total_patches, self.vision_dim, self.mlp_hidden
        attn = sum(4.0 * d * p * p for p in self.seqlens)
        return 8.0 * P * d * d + 6.0 * P * d * h + attn

    def embed_flops(self) -> float:
        return 2.0 * self.total_patches * self.patch_dim * self.vision_dim

    def aligner_flops(self) -> float:
        if not self.aligner:
            return 0.0
        return 2.0 * self.total_patches * self.vision_dim * self.llm_dim

    def total_flops(self) -> float:
        return self.n_blocks * self.block_flops() + self.embed_flops() + self.aligner_flops()


CONFIGS: List[VitConfig] = [
    VitConfig("tiny_fp32_8x8", ((8, 8),), 256, 4, 704, 2, 512, "f32"),
    VitConfig("single_28x28", ((28, 28),), 1024, 16, 2816, 4, 4096, "bf16"),
    VitConfig("ragged_varlen_4img", ((27, 37), (37, 27), (10, 78), (112, 7)),
              1024, 16, 2816, 4, 0, "bf16"),
    VitConfig("highres_64x64_full_tower", ((64, 64),), 1152, 16, 4304, 32, 4096, "bf16"),
    VitConfig("throughput_16x48x48", tuple([(48, 48)] * 16), 1024, 16, 2816, 8, 4096, "bf16"),
]

BY_NAME = {c.name: c for c in CONFIGS}


def get(name_or_index) -> VitConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    return BY_NAME[name_or_index]
