"""Oracle: byte image of the documented cache layout (test infrastructure only).

The layout itself is this library's own choice (the pages fix no byte
format): one slab per (layer, sequence, KV head), each slab a run of 32-token
pages followed, for the KIVI scheme, by the residual ring. Packed b-bit field
i of a run occupies bits [i*b, (i+1)*b), least significant bit of byte 0
first. "K rows" = the page's tokens in order, each token's channels
contiguous; "V cols" = the page's channels in order, each channel's 32 tokens
contiguous.

Every builder returns (bytes, mask): mask has a 1 bit wherever the layout
defines the byte's bit for the tokens the cache holds; bits outside the mask
(unfilled tokens of a partial page, free ring slots) are not specified.

What goes into a page is the encoding of ``codec`` applied exactly as the
pages state it: KIVI keys per channel over the page's 32 tokens and values per
token ("Quantizing the KV cache", going deeper; KIVI How It Works); symmetric
per (token, head) for K and V ("Quantising the Cache.", Workshop); FP8 E4M3
with one scale per KV head ("Quantizing the KV cache", FP8 KV cache).
"""

import numpy as np

from . import codec

PAGE = 32


def pack_fields(codes, bits):
    """Concatenate b-bit fields, field 0 in the lowest bits of byte 0."""
    codes = np.asarray(codes).astype(np.int64).reshape(-1) & ((1 << bits) - 1)
    bit_stream = ((codes[:, None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
    assert bit_stream.size % 8 == 0
    return np.packbits(bit_stream, bitorder="little")


def unpack_fields(buf, bits, n):
    bit_stream = np.unpackbits(np.asarray(buf, np.uint8), bitorder="little")[: n * bits]
    return (bit_stream.reshape(n, bits).astype(np.int64) << np.arange(bits)).sum(axis=1)


def _f32_bytes(x):
    return np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint8).reshape(-1)


def _full(n):
    return np.full(n, 0xFF, np.uint8)


def kivi_page(k32, v32, bits, v_bits=None, outliers=0):
    """One full KIVI page from 32 tokens of keys and values (float32 [32, d]);
    value codes of v_bits when given, else of bits. With outliers == 1 the
    dense-and-sparse encoding (``codec.kivi_quantize_sparse``, one outlier per
    key channel and per value token) and its side matrix after the dense
    page: key outlier values [d] float32, value outlier values [32] float32,
    key outlier tokens [d] uint8, value outlier channels [32] uint8, then
    padding to a multiple of 256 bytes (unspecified)."""
    vb = bits if v_bits is None else v_bits
    d = k32.shape[1]
    if outliers:
        kc, ks, kz, ko, ki = codec.kivi_quantize_sparse(k32, bits, axis=0)
        vc, vs, vz, vo, vi = codec.kivi_quantize_sparse(v32, vb, axis=1)
    else:
        kc, ks, kz = codec.kivi_quantize(k32, bits, axis=0)   # per channel over the tokens
        vc, vs, vz = codec.kivi_quantize(v32, vb, axis=1)     # per token over the channels
    parts = [pack_fields(kc, bits),            # K rows: kc[t, c], channel fastest
             _f32_bytes(ks), _f32_bytes(kz),
             pack_fields(vc.T, vb),            # V cols: vc[t, c] stored channel-major
             _f32_bytes(vs), _f32_bytes(vz)]
    masks = [_full(sum(x.size for x in parts))]
    if outliers:
        side = [_f32_bytes(ko[:, 0]), _f32_bytes(vo[:, 0]),
                ki[:, 0].astype(np.uint8), vi[:, 0].astype(np.uint8)]
        raw = sum(x.size for x in side)
        pad = -(-raw // 256) * 256 - raw
        parts += side + [np.zeros(pad, np.uint8)]
        masks += [_full(raw), np.zeros(pad, np.uint8)]
        assert raw == 5 * d + 5 * PAGE
    buf = np.concatenate(parts)
    return buf, np.concatenate(masks)


def _valid_fields_mask(n_valid, per_row, bits):
    """Mask for `per_row`-field runs whose first n_valid fields are defined."""
    ones = np.where(np.arange(per_row) < n_valid, (1 << bits) - 1, 0)
    return pack_fields(ones, bits)


def sym_page(k32, v32, bits, n_valid):
    """Symmetric page; tokens >= n_valid of k32/v32 are ignored (undefined)."""
    d = k32.shape[1]
    kc, ks = codec.sym_quantize(k32, bits, axis=1)        # one scale per token (K)
    vc, vs = codec.sym_quantize(v32, bits, axis=1)        # one scale per token (V)
    valid = np.arange(PAGE) < n_valid
    kc = np.where(valid[:, None], kc, 0)
    vc = np.where(valid[:, None], vc, 0)
    ks = np.where(valid, ks, np.float32(0))
    vs = np.where(valid, vs, np.float32(0))
    buf = np.concatenate([pack_fields(kc, bits), _f32_bytes(ks),
                          pack_fields(vc.T, bits), _f32_bytes(vs)])
    row = d * bits // 8
    mask = np.concatenate([
        np.repeat(np.where(valid, 0xFF, 0).astype(np.uint8), row),
        np.repeat(np.where(valid, 0xFF, 0).astype(np.uint8), 4),
        np.tile(_valid_fields_mask(n_valid, PAGE, bits), d),
        np.repeat(np.where(valid, 0xFF, 0).astype(np.uint8), 4)])
    return buf, mask


def bf16_page(k32, v32, n_valid):
    """Unquantised page: bfloat16 K rows and V cols (2 bytes per value, least
    significant byte first); tokens >= n_valid undefined."""
    d = k32.shape[1]
    valid = np.arange(PAGE) < n_valid
    kc = np.where(valid[:, None], codec.bf16_encode(k32), 0).astype(np.uint16)
    vc = np.where(valid[:, None], codec.bf16_encode(v32), 0).astype(np.uint16)
    buf = np.concatenate([kc.astype("<u2").view(np.uint8).reshape(-1),
                          np.ascontiguousarray(vc.T).astype("<u2").view(np.uint8).reshape(-1)])
    tok = np.where(valid, 0xFF, 0).astype(np.uint8)
    mask = np.concatenate([np.repeat(tok, 2 * d),            # K rows: a token's 2d bytes
                           np.tile(np.repeat(tok, 2), d)])   # V cols: 2 bytes per token, per channel
    return buf, mask


def fp8_page(k32, v32, k_scale, v_scale, n_valid, fmt="e4m3"):
    """FP8 page (E4M3FN or E5M2) with the KV head's scalar scales; tokens >=
    n_valid undefined. K rows; the values of a full page (n_valid = 32) in V
    cols, those of an open page (the cache's last page while it holds fewer
    than 32 tokens) in rows like the keys, so that a token appended to it
    writes one contiguous row."""
    d = k32.shape[1]
    kc = codec.fp8_quantize(k32, k_scale, fmt)
    vc = codec.fp8_quantize(v32, v_scale, fmt)
    valid = np.arange(PAGE) < n_valid
    kc = np.where(valid[:, None], kc, 0).astype(np.uint8)
    vc = np.where(valid[:, None], vc, 0).astype(np.uint8)
    tok = np.where(valid, 0xFF, 0).astype(np.uint8)
    rows = n_valid < PAGE
    buf = np.concatenate([kc.reshape(-1), vc.reshape(-1) if rows else vc.T.reshape(-1)])
    mask = np.concatenate([np.repeat(tok, d), np.repeat(tok, d) if rows else np.tile(tok, d)])
    return buf, mask


def fp8k_symv_page(k32, v32, k_scale, v_bits, n_valid):
    """Keys and values in different cache types ("Quantizing the KV cache",
    How the KV cache is quantized: separate key and value cache types): the
    key rows of an FP8 E4M3 page with the KV head's scalar key scale, then
    the value columns and per-token value scales of a symmetric page at
    v_bits, then 128 bytes of padding (undefined) that keep the page a
    multiple of 256 bytes; tokens >= n_valid undefined."""
    d = k32.shape[1]
    fb, fm = fp8_page(k32, v32, k_scale, np.float32(1), n_valid, "e4m3")
    sb, sm = sym_page(k32, v32, v_bits, n_valid)
    k_end = PAGE * d                        # FP8 key rows: one byte per value
    v_start = PAGE * d * v_bits // 8 + 4 * PAGE   # after sym_page's key codes and scales
    pad = np.zeros(128, np.uint8)
    return (np.concatenate([fb[:k_end], sb[v_start:], pad]),
            np.concatenate([fm[:k_end], sm[v_start:], pad]))


def fp8k_kiviv_page(k32, v32, k_scale, v_bits, n_valid):
    """FP8 keys with KIVI values ("Quantizing the KV cache", How the KV cache
    is quantized: separate key and value cache types; KIVI How It Works:
    values quantised per token): the key rows of an FP8 E4M3 page with the KV
    head's scalar key scale, then value columns of unsigned v_bits codes, each
    token's value vector encoded by Q_b over its d channels as the KIVI
    page's values are, then the fp32 scale and the fp32 offset (minimum) of
    each token; tokens >= n_valid undefined."""
    d = k32.shape[1]
    fb, fm = fp8_page(k32, v32, k_scale, np.float32(1), n_valid, "e4m3")
    vc, vs, vz = codec.kivi_quantize(v32, v_bits, axis=1)   # per token over the channels
    valid = np.arange(PAGE) < n_valid
    vc = np.where(valid[:, None], vc, 0)
    vs = np.where(valid, vs, np.float32(0))
    vz = np.where(valid, vz, np.float32(0))
    tok = np.repeat(np.where(valid, 0xFF, 0).astype(np.uint8), 4)
    buf = np.concatenate([fb[:PAGE * d], pack_fields(vc.T, v_bits), _f32_bytes(vs), _f32_bytes(vz)])
    mask = np.concatenate([fm[:PAGE * d], np.tile(_valid_fields_mask(n_valid, PAGE, v_bits), d),
                           tok, tok])
    return buf, mask
