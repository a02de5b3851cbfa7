"""Tolerances and comparison helpers for GPU-vs-oracle parity."""
import numpy as np

# bf16 output: max-abs <= 1e-2 and rel-L2 <= 2e-3; fp32 output: both <= 1e-5.
TOL = {"bf16": (1e-2, 2e-3), "f32": (1e-5, 1e-5)}


def errors(gpu: np.ndarray, ref: np.ndarray):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0, 0.0
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    d = g - r
    nr = np.linalg.norm(r)
    return float(np.abs(d).max()), float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d))


def assert_parity(gpu, ref, dtype: str, what: str = ""):
    mx, rel = errors(gpu, ref)
    tol_abs, tol_rel = TOL[dtype]
    print(f"  parity {what}: max_abs={mx:.3e} rel_l2={rel:.3e} ({dtype})", flush=True)
    assert mx <= tol_abs and rel <= tol_rel, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e} over {tol_abs}/{tol_rel}"
    return mx, rel


def to_numpy(t):
    return t.float().cpu().numpy().astype(np.float64)


def storage_bits(t):
    """A device tensor's raw bytes as a numpy array (bf16 -> uint16, fp32 -> float32 bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)
