"""Rotary position embedding in float64 (test infrastructure only).

The pages fix only that every token keeps its original position ID ("Dropping
the Anchor ..." Section 2.1: host i encodes with original position IDs; the
Star Attention review: the anchor keeps its original positional indices).
The rotation itself is the common rotate-half form used by Llama models:
for frequency index i in [0, d/2), inv_freq_i = base ** (-2 i / d), angle
theta = pos * inv_freq_i, and the pair (x_i, x_{i + d/2}) is rotated by theta.
Angles, sines and cosines are float64.
"""
import numpy as np


def inv_freq(head_dim, base):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * i / head_dim)


def rope(x, pos, base):
    """Rotate x[n][H][d] (float64) at positions pos[n]; returns float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(d, base)[None, :]  # [n][d/2]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
