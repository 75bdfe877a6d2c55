"""Plain, slow CPU oracle of the DeepSeek-V4-Flash-Vision encoder hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, tables or helpers); the only thing both sides see
is the seeded input arrays.

Everything is computed with numpy in float64 (pass ``dtype=np.float32`` for the
single-precision reading) as the plain definition of each step, one step after
another, with no blocking, fusion or reordering.  Each function names the page
passage it follows.  Readings taken where the pages are silent or garbled are
listed in ``vit.READINGS``.

Parity pins: every function here is pinned by ``tests/test_oracle.py`` against
closed forms, hand-derived golden values, brute-force loops or invariants.
"""
from .vit import (  # noqa: F401
    NL_END,
    NL_IMAGE,
    NL_NEWLINE,
    NL_START,
    READINGS,
    aligner,
    merge_image_embeddings,
    aligner_gather,
    aligner_perm,
    apply_rope,
    attention,
    attention_probs,
    attn_half_backward,
    block,
    encode,
    encode_varlen,
    gelu,
    layernorm,
    linear,
    mlp,
    mlp_half_backward,
    nlayout,
    patch_embed,
    patch_merger,
    patch_merger_param_count,
    patchify,
    rmsnorm,
    rmsnorm_backward,
    rope_freqs,
    rope_table,
    tower,
    tower_backward,
)
