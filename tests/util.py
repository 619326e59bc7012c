"""Error metrics and helpers shared by the GPU parity tests."""

import numpy as np


def max_abs(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_frob(a, b):
    """||a - b||_F / ||b||_F with b the reference."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def to64(t):
    """A device or host torch tensor as a float64 numpy array."""
    return t.detach().to("cpu").double().numpy()
