"""Rotary position embedding, as the oracle needs it for chunk summaries.

Reading (the pages give no RoPE layout): pairs are half-split, dim i with dim
i + d/2 for i < d/2, with frequency theta_i = base^(-2i/d); position t rotates
pair i by the angle t * theta_i.  Angles are formed in fp64.
"""
import numpy as np


def rope_angles(d, base, pos):
    """angle[..., i] = pos * base^(-2i/d) for i < d/2 (fp64)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return np.asarray(pos, np.float64)[..., None] * theta


def rope_rotate(x, angle):
    """Rotate the (i, i + d/2) pairs of x[..., d] by angle[..., i]."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = np.cos(angle), np.sin(angle)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
