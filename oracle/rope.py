"""Rotary position embedding in float64 (test infrastructure only).

The pages fix only that every token keeps its original position ID ("Dropping
the Anchor ..." Section 2.1: host i encodes with original position IDs; the
Star Attention review: the anchor keeps its original positional indices).
The rotation itself is the common rotate-half form used by Llama models:
for frequency index i in [0, d/2), inv_freq_i = base ** (-2 i / d), angle
theta = pos * inv_freq_i, and the pair (x_i, x_{i + d/2}) is rotated by theta.
Angles, sines and cosines are float64.

Llama-3.1 checkpoints (the model of the pages' experiments) rescale these
frequencies; the published rule ("llama3" rope scaling: factor 8, low- and
high-frequency factors 1 and 4, original context 8192) keeps frequencies whose
wavelength 2 pi / f is shorter than 8192 / 4 positions, divides those longer
than 8192 / 1 by 8, and between the two blends f / 8 and f linearly in
8192 / wavelength.  A base wrapped in Llama3Base selects it.
"""
import numpy as np


class Llama3Base(float):
    """A RoPE base number that also selects the Llama-3.1 frequency scaling."""


def _llama3(f):
    factor, low, high, orig = 8.0, 1.0, 4.0, 8192.0
    wavelen = 2.0 * np.pi / f
    smooth = (orig / wavelen - low) / (high - low)
    mid = (1.0 - smooth) * f / factor + smooth * f
    return np.where(wavelen < orig / high, f, np.where(wavelen > orig / low, f / factor, mid))


def inv_freq(head_dim, base):
    i = np.arange(head_dim // 2, dtype=np.float64)
    f = float(base) ** (-2.0 * i / head_dim)
    return _llama3(f) if isinstance(base, Llama3Base) else f


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
