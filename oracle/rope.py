"""RoPE and RoPE relocation, fp64.

Pages: RedKnot README (topairepos.com), "About" (offline KV reuse + RoPE
relocation "guarantees numerical alignment") and "Key Ideas" (rope_helper);
aitrends.kr "주요 기능" (stored KV is re-aligned to the current positions).

Reading (the pages give no formula): rotate-half (NeoX) pairing of dimension j
with j + D/2, frequency omega_j = theta ** (-2j/D) over the full head
dimension. A vector at position p has each pair rotated by angle p * omega_j.
Relocating cached K from original position o to new position b is rotation by
delta = b - o, because rotations by p and then delta compose to p + delta.
"""
import numpy as np


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * j / head_dim)


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate x[..., D] at positions ``pos`` (broadcast over x's leading dims)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def relocate(k_cached: np.ndarray, delta, theta: float) -> np.ndarray:
    """Move cached K from its original positions by ``delta`` tokens."""
    return rope(k_cached, delta, theta)
