"""Write the oracle's expected outputs for the workloads too large to run the
oracle inside a GPU test.  Calls only ``oracle`` (and the seeded input
generator); nothing here touches the HIP path.

    python tests/golden/make_expected.py highres_64x64_full_tower

Stores every output row (float32) plus a fingerprint of the inputs in
``tests/golden/expected_<workload>.npz``.
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from vision_transformer_encoder_image_amd import configs, synth  # noqa: E402

ROW_STRIDE = 1


def fingerprint(inp) -> str:
    h = hashlib.sha256()
    h.update(inp["patches"].tobytes())
    w = inp["weights"]
    h.update(w["patch_embed"].tobytes())
    for b in w["blocks"]:
        for k in sorted(b):
            h.update(b[k].tobytes())
    h.update(w["final_norm"].tobytes())
    if w["aligner"] is not None:
        h.update(w["aligner"].tobytes())
    return h.hexdigest()


def main(name: str) -> None:
    idx = [c.name for c in configs.CONFIGS].index(name)
    cfg = configs.CONFIGS[idx]
    inp = synth.make_inputs(cfg, seed=idx)
    t0 = time.time()
    out = oracle.encode_varlen(inp["patches"], inp["grids"], inp["weights"], cfg.n_heads,
                               cfg.rms_eps, cfg.rope_theta, with_aligner=cfg.aligner)
    rows = np.arange(0, out.shape[0], ROW_STRIDE)
    path = os.path.join(ROOT, "tests", "golden", f"expected_{name}.npz")
    np.savez_compressed(path, rows=rows.astype(np.int64), values=out[rows].astype(np.float32),
                        shape=np.array(out.shape, dtype=np.int64),
                        fingerprint=np.array(fingerprint(inp)), seed=np.array(idx))
    print(f"{name}: oracle {time.time() - t0:.1f}s, wrote {path} ({len(rows)} rows)")


if __name__ == "__main__":
    for n in sys.argv[1:]:
        main(n)
