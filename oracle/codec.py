"""Oracle: the three cache encodings and their decodings (test infrastructure only).

All encoding arithmetic is IEEE float32 (numpy float32 arrays), in the order
the formulas are written, with true division and ties-to-even rounding
(``np.rint``); decodings are float64.

* ``kivi_quantize`` -- "Quantizing the KV cache", going deeper ("Per-channel
  and per-token grouping"): Q_b(x) = round((x - min x)/s) * s + min x with
  s = (max x - min x)/(2^b - 1), asymmetric, one (s, min) per group. Keys are
  grouped per channel over a block of tokens, values per token ("Keys and
  values are shaped differently"; KIVI How It Works).
  Readings where the page is silent: ``round`` is ties-to-even; s == 0 (a
  constant group) gives code 0 and the group decodes to its minimum exactly;
  a minimum of -0 is stored as +0.
* ``sym_quantize`` -- "Quantising the Cache.", Workshop: symmetric
  round-to-nearest of each head's key and value at every token. Reading: the
  grid is s * {-Q..Q}, Q = 2^(b-1) - 1, s = max|x| / Q.
* ``e4m3_encode`` / ``e4m3_decode`` -- "Quantizing the KV cache", "How the KV
  cache is quantized": FP8 (E4M3) cache with per-head scales. Reading: the OCP
  E4M3FN format (exponent bias 7, no infinities, S.1111.111 is NaN, largest
  finite 448); a value goes to the nearest finite E4M3 number, ties to the
  even code, so anything beyond 448 saturates to 448; the sign is kept.
* ``e5m2_encode`` / ``e5m2_decode`` -- the other FP8 format the same section
  names ("E4M3 or E5M2"). Reading: OCP E5M2 (exponent bias 15, S.11111.00 is
  infinity, S.11111.xx NaN, largest finite 57344); nearest finite value, ties
  to the even code, beyond 57344 saturated (as for E4M3: no infinities are
  produced); the sign is kept.
* ``bf16_encode`` / ``bf16_decode`` -- the unquantised 16-bit cache that the
  pages measure the others against ("Quantizing the KV cache", "The other big
  memory user": two bytes per value). Reading: bfloat16 (the top 16 bits of a
  float32), float32 input rounded to the nearest bfloat16, ties to the even
  pattern.
"""

import numpy as np

F32 = np.float32


def kivi_quantize(x, bits, axis):
    """Asymmetric b-bit round-to-nearest of `x` (float32) in groups along `axis`.

    Returns (codes uint8 with the same shape as x, s float32, z float32) where
    s and z have `axis` removed. Decoding: code * s + z."""
    x = np.asarray(x, dtype=F32)
    levels = F32(2 ** bits - 1)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    mn = mn + F32(0.0)                         # -0 -> +0
    s = (mx - mn) / levels                     # float32 / float32
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((x - mn) / s)              # ties to even
    r = np.where(s == 0, F32(0.0), r)          # constant group: code 0
    codes = np.clip(r, F32(0.0), levels).astype(np.uint8)
    return codes, np.squeeze(s, axis=axis), np.squeeze(mn, axis=axis)


def kivi_quantize_sparse(x, bits, axis, n_out=1):
    """Dense-and-sparse KIVI quantisation ("KVQuant: Towards 10 Million Context
    Length ...", Summary: a small fraction of outliers moved, per vector, into
    a separate sparse representation; "Quantizing the KV cache", going deeper:
    KVQuant keeps a few outliers in a sparse side matrix).

    Reading: each vector along `axis` (a key channel's tokens of one group, a
    value token's channels) moves its n_out values of largest magnitude |x|
    (equal magnitudes: the lower index first) into the side matrix, stored
    exactly with their index; the other values are quantised by Q_b exactly as
    ``kivi_quantize`` does, with min and max taken over those values only; the
    moved positions hold code 0.

    Returns (codes, s, z, out_val, out_idx): codes like ``kivi_quantize``; s,
    z with `axis` removed; out_val float32 and out_idx int64 with `axis`
    replaced by a last axis of length n_out (in the selection order)."""
    x = np.moveaxis(np.asarray(x, dtype=F32), axis, -1)
    n = x.shape[-1]
    assert 0 < n_out < n
    order = np.argsort(-np.abs(x), axis=-1, kind="stable")   # ties: lower index first
    out_idx = order[..., :n_out]
    out_val = np.take_along_axis(x, out_idx, axis=-1)
    moved = np.zeros(x.shape, bool)
    np.put_along_axis(moved, out_idx, True, axis=-1)
    levels = F32(2 ** bits - 1)
    mn = np.where(moved, F32(np.inf), x).min(axis=-1, keepdims=True)
    mx = np.where(moved, F32(-np.inf), x).max(axis=-1, keepdims=True)
    mn = mn + F32(0.0)                         # -0 -> +0
    s = (mx - mn) / levels
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint((x - mn) / s)
    r = np.where(s == 0, F32(0.0), r)
    r = np.where(moved, F32(0.0), r)           # moved positions: code 0
    codes = np.clip(r, F32(0.0), levels).astype(np.uint8)
    return (np.moveaxis(codes, -1, axis), np.squeeze(s, -1), np.squeeze(mn, -1),
            out_val, out_idx)


def kivi_dequantize_sparse(codes, s, z, out_val, out_idx, axis):
    """Dense dequantisation code * s + z (float64) with the side matrix's
    values put back exactly at their positions."""
    x = np.moveaxis(kivi_dequantize(codes, s, z, axis), axis, -1).copy()
    np.put_along_axis(x, np.asarray(out_idx), np.asarray(out_val, np.float64), axis=-1)
    return np.moveaxis(x, -1, axis)


def kivi_dequantize(codes, s, z, axis):
    """code * s + z in float64, s and z broadcast back along `axis`."""
    s64 = np.expand_dims(np.asarray(s, np.float64), axis)
    z64 = np.expand_dims(np.asarray(z, np.float64), axis)
    return np.asarray(codes, np.float64) * s64 + z64


def sym_quantize(x, bits, axis):
    """Symmetric b-bit round-to-nearest with one scale per group along `axis`.

    Returns (codes int8 in [-Q, Q], s float32 with `axis` removed)."""
    x = np.asarray(x, dtype=F32)
    qmax = F32(2 ** (bits - 1) - 1)
    a = np.abs(x).max(axis=axis, keepdims=True)
    s = a / qmax
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(x / s)
    r = np.where(s == 0, F32(0.0), r)
    codes = np.clip(r, -qmax, qmax).astype(np.int8)
    return codes, np.squeeze(s, axis=axis)


def sym_dequantize(codes, s, axis):
    return np.asarray(codes, np.float64) * np.expand_dims(np.asarray(s, np.float64), axis)


# ---- FP8 E4M3FN -------------------------------------------------------------

def e4m3_value(code):
    """Value of one E4M3FN byte by its definition (sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 is subnormal; 0x7F/0xFF are NaN)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# Finite non-negative magnitudes are codes 0x00..0x7E, increasing with the code.
_MAGS = E4M3_TABLE[:0x7F]


def e4m3_encode(y):
    """Nearest finite E4M3FN number to each float32 `y`, ties to the even code
    (even mantissa), beyond 448 saturated, sign bit copied from y."""
    y = np.asarray(y, dtype=F32)
    a = np.abs(y).astype(np.float64)                   # exact
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 0, len(_MAGS) - 1)
    lo = np.clip(hi - 1, 0, len(_MAGS) - 1)
    d_hi = np.abs(_MAGS[hi] - a)
    d_lo = np.abs(a - _MAGS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    pick_lo &= a <= _MAGS[-1]            # beyond the largest finite value: saturate
    mag = np.where(pick_lo, lo, hi).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e4m3_encode_bruteforce(y):
    """Same rule by a full scan of all 127 finite magnitudes (small inputs)."""
    out = []
    for v in np.asarray(y, dtype=F32).reshape(-1):
        a = min(abs(float(v)), 448.0)            # saturation, then the nearest of all
        best, best_d = None, None
        for c in range(0x7F):
            d = abs(E4M3_TABLE[c] - a)
            if best is None or d < best_d or (d == best_d and c % 2 == 0 and best % 2 == 1):
                best, best_d = c, d
        out.append(best | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(y))


def e4m3_decode(codes):
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ---- FP8 E5M2 ----------------------------------------------------------------

def e5m2_value(code):
    """Value of one E5M2 byte by its definition (sign, 5-bit exponent with bias
    15, 2-bit mantissa; exponent 0 is subnormal; exponent 31 is inf / NaN)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (m / 4.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)
# Finite non-negative magnitudes are codes 0x00..0x7B, increasing with the code.
_MAGS5 = E5M2_TABLE[:0x7C]


def e5m2_encode(y):
    """Nearest finite E5M2 number to each float32 `y`, ties to the even code,
    beyond 57344 saturated, sign bit copied from y."""
    y = np.asarray(y, dtype=F32)
    a = np.abs(y).astype(np.float64)
    hi = np.clip(np.searchsorted(_MAGS5, a, side="left"), 0, len(_MAGS5) - 1)
    lo = np.clip(hi - 1, 0, len(_MAGS5) - 1)
    d_hi = np.abs(_MAGS5[hi] - a)
    d_lo = np.abs(a - _MAGS5[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    pick_lo &= a <= _MAGS5[-1]           # beyond the largest finite value: saturate
    mag = np.where(pick_lo, lo, hi).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e5m2_encode_bruteforce(y):
    """Same rule by a full scan of all 124 finite magnitudes (small inputs)."""
    out = []
    for v in np.asarray(y, dtype=F32).reshape(-1):
        a = min(abs(float(v)), 57344.0)          # saturation, then the nearest of all
        best, best_d = None, None
        for c in range(0x7C):
            d = abs(E5M2_TABLE[c] - a)
            if best is None or d < best_d or (d == best_d and c % 2 == 0 and best % 2 == 1):
                best, best_d = c, d
        out.append(best | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(y))


def e5m2_decode(codes):
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp8_quantize(x, scale, fmt="e4m3"):
    """FP8(x / scale) with a float32 scale per KV head (broadcast), E4M3FN or E5M2."""
    x = np.asarray(x, dtype=F32)
    y = x / np.asarray(scale, dtype=F32)
    return e5m2_encode(y) if fmt == "e5m2" else e4m3_encode(y)


def fp8_dequantize(codes, scale, fmt="e4m3"):
    vals = e5m2_decode(codes) if fmt == "e5m2" else e4m3_decode(codes)
    return vals * np.asarray(scale, np.float64)


# ---- bfloat16 ---------------------------------------------------------------

def bf16_encode(x):
    """bfloat16 patterns (uint16) nearest to the finite float32 values `x`.

    The two bfloat16 neighbours of a float32 are its top 16 bits (toward zero)
    and that pattern plus one (away from zero); the dropped low 16 bits say
    how far x is past the first: below half a unit keep it, above take the
    next, exactly half take whichever pattern is even."""
    bits = np.asarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    keep = bits >> 16
    dropped = bits & 0xFFFF
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((keep & 1) == 1))
    return (keep + up).astype(np.uint16)


def bf16_decode(codes):
    """Exact float64 values of bfloat16 patterns."""
    raw = np.asarray(codes, np.uint16).astype(np.uint32) << 16
    return raw.view(np.float32).astype(np.float64)
