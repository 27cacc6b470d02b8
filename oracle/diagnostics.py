"""Diagnostics of the quantization scheme (numpy, fp64) -- TEST INFRASTRUCTURE ONLY.

These reproduce, on synthetic inputs, the quantities the two-panel figure of
"int8 Flash Attention on RDNA4: QK Wants Integers, PV Wants FP8" measures:

* left panel: where an attention row keeps its probability mass, by magnitude
  decade, and how much of it falls below int8's round-to-zero threshold
  0.5/127 (static P scale 127);
* right panel: per-channel absmax of K relative to the median channel, before
  and after subtracting the per-channel mean, and the int8 levels a per-tensor
  scale leaves to the typical channel (127 * median / max).
"""
from __future__ import annotations

import numpy as np

DECADE_EDGES = np.array([0.0, 1e-4, 1e-3, 1e-2, 1e-1, 1.0 + 1e-12])
INT8_ZERO_THRESHOLD = 0.5 / 127.0


def softmax_rows(scores: np.ndarray) -> np.ndarray:
    s = scores - scores.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def mass_by_decade(p: np.ndarray) -> np.ndarray:
    """Fraction of total probability mass in [0,1e-4), [1e-4,1e-3), [1e-3,1e-2),
    [1e-2,1e-1), [1e-1,1], averaged over rows. p: [rows][keys], rows sum to 1."""
    out = np.zeros(len(DECADE_EDGES) - 1)
    for i in range(len(out)):
        sel = (p >= DECADE_EDGES[i]) & (p < DECADE_EDGES[i + 1])
        out[i] = np.mean(np.sum(np.where(sel, p, 0.0), axis=-1))
    return out


def mass_below(p: np.ndarray, threshold: float = INT8_ZERO_THRESHOLD) -> float:
    return float(np.mean(np.sum(np.where(p < threshold, p, 0.0), axis=-1)))


def gaussian_logit_rows(rng: np.random.Generator, rows: int, keys: int, std: float) -> np.ndarray:
    """Rows of softmax weights from Gaussian logits of the given std."""
    return softmax_rows(std * rng.standard_normal((rows, keys)))


def channel_absmax_ratios(k: np.ndarray, centred: bool) -> np.ndarray:
    """k: [N][d] -> per-channel absmax / median channel absmax."""
    x = k.astype(np.float64)
    if centred:
        x = x - x.mean(axis=0, keepdims=True)
    a = np.abs(x).max(axis=0)
    return a / np.median(a)


def typical_channel_levels(k: np.ndarray, centred: bool) -> float:
    """int8 levels a single per-tensor scale leaves to the median channel."""
    r = channel_absmax_ratios(k, centred)
    return 127.0 / r.max()
