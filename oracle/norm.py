"""Per-head QK-RMSNorm, float64.

Source: "Qwen3-4B" page, the QK-norm paragraph: an RMS normalization of
every head's head_dim-wide slice of the query and key projections, applied
after the split into heads and before rope, with its own gain vector of
width head_dim for queries and for keys, epsilon 1e-6; normalizing the
flattened Heads*HeadDim projection instead is called out there as wrong.

Reading (the norm body is not shown on the pages): the usual RMSNorm,
y = g * x / sqrt(mean(x**2) + eps), epsilon inside the square root, gain
applied after normalizing.
"""
import numpy as np


def rms_norm_heads(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x: [..., D] float64 (the last axis is one head's slice); gain: [D]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gain, dtype=np.float64) * x / np.sqrt(ms + eps)
