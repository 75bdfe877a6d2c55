"""Error measures shared by the GPU parity tests (host side, float64)."""
import numpy as np

# Bars for the whole encoder: max row-wise relative error 2e-2 in bf16, 1e-4 in fp32.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rowwise_rel_err(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def global_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def frob_rel_err(got, ref):
    """||got - ref||_F / ||ref||_F over the whole array (float64)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
