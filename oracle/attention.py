"""Oracle: decode attention by its definition, float64 (test infrastructure only).

"Quantizing the KV cache", going deeper ("Why values per token"): the output
for a query is o = sum_t p_t V_t with attention weights p_t, the keys entering
through the dot products q . K_t. Readings where the page is silent: p is the
textbook softmax of sm_scale * q . K_t over every cached token (no mask), with
sm_scale = 1/sqrt(head_dim) unless given; query head h reads KV head
floor(h / (q_heads / kv_heads)) ("Quantizing the KV cache": grouped-query
attention shares each key/value head among several query heads).
"""

import math

import numpy as np


def attend(q, k, v, sm_scale):
    """One query row against T keys/values, all float64.

    q [d], k [T, d], v [T, d] -> o [d]."""
    q = np.asarray(q, np.float64)
    s = sm_scale * (np.asarray(k, np.float64) @ q)
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ np.asarray(v, np.float64)


def attend_bruteforce(q, k, v, sm_scale):
    """Same definition with Python loops and math.exp (tiny inputs only)."""
    T, d = len(k), len(q)
    scores = [sm_scale * sum(float(q[c]) * float(k[t][c]) for c in range(d)) for t in range(T)]
    m = max(scores)
    w = [math.exp(x - m) for x in scores]
    tot = sum(w)
    return np.array([sum(w[t] * float(v[t][c]) for t in range(T)) / tot for c in range(d)])


def gqa_kv_head(h, q_heads, kv_heads):
    return h // (q_heads // kv_heads)


def decode(q, khat, vhat, sm_scale):
    """Decode attention for every (sequence, query head).

    q [B, Hq, d]; khat, vhat [B, Hkv, T, d] (dequantised, already rotated if
    the rotary embedding is on) -> out [B, Hq, d] float64."""
    B, Hq, d = q.shape
    Hkv = khat.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            g = gqa_kv_head(h, Hq, Hkv)
            out[b, h] = attend(q[b, h], khat[b, g], vhat[b, g], sm_scale)
    return out


def split_merge(q, k, v, sm_scale, bounds):
    """The same result assembled from token chunks [bounds[i], bounds[i+1]):
    each chunk keeps (max score m, sum of exp l, unnormalised sum o); chunks
    combine as M = max m_i, o = sum e^(m_i-M) o_i / sum e^(m_i-M) l_i. This is
    algebraically identical to ``attend`` and is used to pin the GPU's merge
    step's arithmetic."""
    q = np.asarray(q, np.float64)
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b <= a:
            continue
        s = sm_scale * (np.asarray(k[a:b], np.float64) @ q)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ np.asarray(v[a:b], np.float64)))
    M = max(m for m, _, _ in parts)
    num = sum(math.exp(m - M) * o for m, _, o in parts)
    den = sum(math.exp(m - M) * l for m, l, _ in parts)
    return num / den
