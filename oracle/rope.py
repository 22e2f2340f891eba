"""Rotary positions: frequency table and rotation, in float64.

Sources:
- "Phi-3 Mini 4K Instruct" files, src/rope.linnet (`tables`): frequency i of
  a head of width D is theta ** (-2i/D) for i < D/2 (written there as
  exp(-(2i/D) ln theta)); the angle at position s is s * f[i]; the angle
  table is concatenated with itself so each frequency serves both halves of
  the head vector.
- "Llama 3.1 8B Instruct", rope scaling paragraph and Validation: per
  frequency, by wavelength 2*pi/f: longer than original/low_freq_factor ->
  divided by factor; shorter than original/high_freq_factor -> unchanged;
  in between -> linear blend (1 - s) * f / factor + s * f, with s = 1 at the
  short-wavelength boundary (continuity with the unchanged band).

Readings where the pages are silent:
- pairing: rotate-half, dimension i with i + D/2 (what the duplicated
  [angles, angles] table implies);
- blend weight: s = (original / wavelength - low_freq_factor) /
  (high_freq_factor - low_freq_factor), linear in frequency; it is 1 at
  wavelength original/high_freq_factor and 0 at original/low_freq_factor,
  matching both band edges;
- cos/sin are exact float64 functions of the float64 angle (the pages cast
  their tables to the model dtype; that rounding is not reproduced).
"""
import math

import numpy as np


def inv_freq(theta: float, head_dim: int, llama3=None) -> np.ndarray:
    """Frequency table f[i], i < head_dim/2, float64.

    llama3 = (factor, low_freq_factor, high_freq_factor, original_max_position)
    or None."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    f = np.power(float(theta), -2.0 * i / head_dim)
    if llama3 is None:
        return f
    factor, low_ff, high_ff, original = (float(v) for v in llama3)
    low_freq_wavelen = original / low_ff      # 8192 for Llama 3.1
    high_freq_wavelen = original / high_ff    # 2048 for Llama 3.1
    out = np.empty_like(f)
    for k in range(f.shape[0]):
        wavelen = 2.0 * math.pi / f[k]
        if wavelen < high_freq_wavelen:
            out[k] = f[k]
        elif wavelen > low_freq_wavelen:
            out[k] = f[k] / factor
        else:
            s = (original / wavelen - low_ff) / (high_ff - low_ff)
            out[k] = (1.0 - s) * f[k] / factor + s * f[k]
    return out


def rotate(x: np.ndarray, positions, freqs: np.ndarray) -> np.ndarray:
    """Rotate head vectors by their token's position.

    x: [T, n_heads, D] float64; positions: [T] integers; freqs: [D/2].
    For each pair (i, i + D/2) with angle a = p * f[i]:
        y[i]       = x[i] cos a - x[i + D/2] sin a
        y[i + D/2] = x[i + D/2] cos a + x[i] sin a
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    p = np.asarray(positions, dtype=np.float64)
    angle = p[:, None] * freqs[None, :]                 # [T, D/2]
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
