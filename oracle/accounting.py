"""Oracle: memory accounting of the KV cache (test infrastructure only).

* ``kv_bytes_formula`` -- "Quantizing the KV cache", section "The other big
  memory user": KV bytes = 2 x layers x KV heads x head size x tokens x bytes
  per value, the 2 counting keys and values. With keys and values stored at
  different widths (the same page's "How the KV cache is quantized" names
  separate key and value cache types) each half counts at its own width.
* ``concurrency`` -- "Quantising the Cache.", Workshop and "Twice the users for
  nearly nothing": how many 8192-token conversations fit beside Llama 3 8B's
  16.1 GB of BF16 weights on an 80 GB GPU used to 90%, cache scales ignored.
* ``layout_cache_bytes`` -- the byte size of the documented cache layout
  (pages of 32 tokens per (layer, sequence, KV head), plus the residual ring
  for the KIVI scheme), computed here from that description alone.
"""

from fractions import Fraction

KIVI, SYM_TOKEN, FP8_E4M3, BF16_CACHE, FP8_E5M2, FP8K_SYMV, FP8K_KIVIV = 0, 1, 2, 3, 4, 5, 6
PAGE = 32


def kv_bytes_formula(layers, kv_heads, head_dim, tokens, bits, batch=1, v_bits=None):
    """2 * layers * kv_heads * head_dim * tokens * bits/8 (times sequences);
    with v_bits, layers * kv_heads * head_dim * tokens * (bits + v_bits)/8.

    Exact integer arithmetic (bits/8 kept as a fraction, so 4-bit works)."""
    vb = bits if v_bits is None else v_bits
    b = Fraction(layers * kv_heads * head_dim * tokens * batch) * Fraction(bits + vb, 8)
    assert b.denominator == 1, "bytes must be whole"
    return int(b)


def concurrency(bits, gpu_bytes=80e9, use=0.9, weight_bytes=16.1e9,
                context=8192, layers=32, kv_heads=8, head_dim=128):
    """Conversations of `context` tokens that fit in the memory left beside
    the weights: floor((use*gpu - weights) / (context * bytes per token)).
    Llama 3 8B shape (32 layers, 8 KV heads of 128), scales ignored."""
    per_token = kv_bytes_formula(layers, kv_heads, head_dim, 1, bits)
    free = use * gpu_bytes - weight_bytes
    return int(free // (context * per_token))


def flush_plan(tokens, residual, group=PAGE):
    """Split of a T-token KIVI cache into quantised and full-precision parts.

    The newest `residual` tokens always stay in full precision; whenever the
    unquantised tokens reach residual+group, the oldest `group` of them are
    encoded together ("Quantizing the KV cache": the window is quantised as a
    group once it fills, and a recent window of R tokens is never rounded;
    KIVI How It Works: the most recent tokens kept unquantised).
    Returns (q, n_r): q tokens in quantised groups, n_r = T - q unquantised."""
    q = group * (max(0, tokens - residual) // group)
    return q, tokens - q


def sparse_section_bytes(head_dim):
    """The side matrix of one KIVI page with one outlier per vector: the key
    outlier of each channel (float32) and the value outlier of each token
    (float32), then their indices (one byte each: token 0..31, channel
    0..d-1), padded to a multiple of 256 bytes."""
    raw = 4 * head_dim + 4 * PAGE + head_dim + PAGE
    return -(-raw // 256) * 256


def page_bytes(scheme, head_dim, bits, v_bits=None, outliers=0):
    """Bytes of one 32-token page of the documented layout (KIVI value codes
    of v_bits when given, else of bits; with the sparse side matrix of one
    outlier per vector when outliers == 1)."""
    d, b = head_dim, bits
    vb = bits if v_bits is None else v_bits
    if scheme == KIVI:
        # K codes + K scale/offset per channel + V codes + V scale/offset per token
        base = PAGE * d * b // 8 + 4 * d + 4 * d + PAGE * d * vb // 8 + 4 * PAGE + 4 * PAGE
        return base + (sparse_section_bytes(d) if outliers else 0)
    assert not outliers
    if scheme == SYM_TOKEN:
        return PAGE * d * b // 8 + 4 * PAGE + PAGE * d * b // 8 + 4 * PAGE
    if scheme in (FP8_E4M3, FP8_E5M2):
        return PAGE * d + PAGE * d
    if scheme == BF16_CACHE:
        return PAGE * d * 2 + PAGE * d * 2      # 16-bit K rows + V cols
    if scheme == FP8K_SYMV:
        # FP8 K rows + symmetric V codes at v_bits + one V scale per token,
        # the scales padded to 256 bytes (pages stay 256-byte multiples)
        return PAGE * d + PAGE * d * vb // 8 + 256
    if scheme == FP8K_KIVIV:
        # FP8 K rows + KIVI V codes at v_bits + V scale and offset per token
        return PAGE * d + PAGE * d * vb // 8 + 4 * PAGE + 4 * PAGE
    raise ValueError(scheme)


def pages_per_slab(scheme, capacity, residual):
    if scheme == KIVI:
        return max(0, capacity - residual) // PAGE
    return -(-capacity // PAGE)


def ring_bytes(scheme, head_dim, residual, in_itemsize):
    if scheme != KIVI:
        return 0
    return 2 * (residual + PAGE) * head_dim * in_itemsize


def slab_bytes(scheme, head_dim, bits, capacity, residual, in_itemsize, v_bits=None, outliers=0):
    return (pages_per_slab(scheme, capacity, residual)
            * page_bytes(scheme, head_dim, bits, v_bits, outliers)
            + ring_bytes(scheme, head_dim, residual, in_itemsize))


def layout_cache_bytes(scheme, layers, batch, kv_heads, head_dim, bits, capacity,
                       residual, in_itemsize, v_bits=None, outliers=0):
    """Whole cache: one slab per (layer, sequence, KV head)."""
    return layers * batch * kv_heads * slab_bytes(scheme, head_dim, bits, capacity,
                                                  residual, in_itemsize, v_bits, outliers)
