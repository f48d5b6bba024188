"""Oracle: rotary position embedding in float64 (test infrastructure only).

"KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (Summary): keys are quantised before the rotary embedding,
which mixes channel pairs, so the rotation is applied after dequantisation.
The rotation is the RoFormer one (cited in KVQuant's reference list):
channel pair (2i, 2i+1) at position p is turned by the angle
p * theta^(-2i/d):   (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
Reading: no frequency scaling; angles formed in float64.
"""

import numpy as np


def frequencies(head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rotate(x, positions, theta):
    """Rotate the last axis (head_dim) of `x` ([..., n, d] with one position per
    row, or [..., d] with a scalar position) by the rotary embedding."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    w = frequencies(d, theta)
    pos = np.asarray(positions, np.float64)
    ang = pos[..., None] * w                       # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
