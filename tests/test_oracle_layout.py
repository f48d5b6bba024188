"""Pins of oracle.layout and oracle.cache: bit packing by hand, page contents
decoded back, the flush rule, and chunking independence."""

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import codec, layout
from oracle.cache import OracleCache, bf16_bits_to_f32

F32 = np.float32


def test_pack_fields_by_hand():
    # 2-bit fields 1,2,3,0 -> 0b00_11_10_01
    assert layout.pack_fields([1, 2, 3, 0], 2).tolist() == [0b00111001]
    # 4-bit fields 0xA, 0x5, 0xF, 0x1 -> bytes 0x5A, 0x1F
    assert layout.pack_fields([0xA, 0x5, 0xF, 0x1], 4).tolist() == [0x5A, 0x1F]
    assert layout.pack_fields([7, 200], 8).tolist() == [7, 200]
    # two's complement 4-bit: -1 -> 0xF, -7 -> 0x9
    assert layout.pack_fields([-1, -7], 4).tolist() == [0x9F]
    rng = np.random.default_rng(0)
    for b in (2, 4, 8):
        c = rng.integers(0, 2 ** b, 256)
        assert np.array_equal(layout.unpack_fields(layout.pack_fields(c, b), b, 256), c)


def test_bf16_bits():
    assert bf16_bits_to_f32(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16)).tolist() == \
        [1.0, -2.0, 0.0, -0.0]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_kivi_page_roundtrip(bits):
    rng = np.random.default_rng(bits)
    d = 64
    k = rng.standard_normal((32, d)).astype(F32)
    v = rng.standard_normal((32, d)).astype(F32)
    buf, mask = layout.kivi_page(k, v, bits)
    assert buf.size == acc.page_bytes(acc.KIVI, d, bits) and np.all(mask == 0xFF)
    nb = 32 * d * bits // 8
    kc = layout.unpack_fields(buf[:nb], bits, 32 * d).reshape(32, d)
    ks = buf[nb:nb + 4 * d].view(F32)
    kz = buf[nb + 4 * d:nb + 8 * d].view(F32)
    o = nb + 8 * d
    vcols = layout.unpack_fields(buf[o:o + nb], bits, 32 * d).reshape(d, 32)
    vs = buf[o + nb:o + nb + 128].view(F32)
    vz = buf[o + nb + 128:o + nb + 256].view(F32)
    # keys: one scale per channel; values: one per token
    assert np.array_equal(kz, k.min(axis=0)) and np.array_equal(vz, v.min(axis=1))
    kh = kc * ks.astype(np.float64) + kz
    vh = vcols.T * vs.astype(np.float64)[:, None] + vz[:, None]
    assert np.all(np.abs(kh - k) <= ks / 2 * (1 + 1e-5))
    assert np.all(np.abs(vh - v) <= vs[:, None] / 2 * (1 + 1e-5))
    # an element in token 3, channel 5 sits at field 3*d+5 (K) and 5*32+3 (V)
    c, s, z = codec.kivi_quantize(k, bits, axis=0)
    assert kc[3, 5] == c[3, 5]
    c, s, z = codec.kivi_quantize(v, bits, axis=1)
    assert vcols[5, 3] == c[3, 5]


def test_sym_and_fp8_partial_page_masks():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((32, 32)).astype(F32)
    v = rng.standard_normal((32, 32)).astype(F32)
    buf, mask = layout.sym_page(k, v, 4, 5)
    assert buf.size == mask.size == acc.page_bytes(acc.SYM_TOKEN, 32, 4)
    row = 32 * 4 // 8
    assert np.all(mask[:5 * row] == 0xFF) and np.all(mask[5 * row:32 * row] == 0)
    kc = layout.unpack_fields(buf[:5 * row], 4, 5 * 32)
    kc = np.where(kc > 7, kc - 16, kc).reshape(5, 32)
    c, s = codec.sym_quantize(k[:5], 4, axis=1)
    assert np.array_equal(kc, c)
    # V cols: first 5 of each channel's 32 four-bit fields defined -> 0xFF,0xFF,0x0F,0...
    vmask = mask[32 * row + 128: 32 * row + 128 + 16]
    assert vmask.tolist() == [0xFF, 0xFF, 0x0F] + [0] * 13
    # open FP8 page (31 tokens): K rows and V rows (token 30's 32 value bytes
    # contiguous, token 31's undefined)
    buf, mask = layout.fp8_page(k, v, F32(0.5), F32(2.0), 31)
    assert buf.size == 2048 and mask.sum() == 0xFF * 31 * 32 * 2
    assert mask[32 * 31 + 1] == 0 and mask[32 * 30 + 1] == 0xFF
    assert buf[32 * 30 + 1] == codec.fp8_quantize(k[30, 1], F32(0.5))
    assert buf[1024 + 30 * 32 + 7] == codec.fp8_quantize(v[30, 7], F32(2.0))
    assert np.all(mask[1024 + 30 * 32:1024 + 31 * 32] == 0xFF) and np.all(mask[1024 + 31 * 32:] == 0)
    # full page: V cols (channel 7's 32 tokens contiguous)
    buf, mask = layout.fp8_page(k, v, F32(0.5), F32(2.0), 32)
    assert np.all(mask == 0xFF)
    assert buf[1024 + 7 * 32 + 30] == codec.fp8_quantize(v[30, 7], F32(2.0))
    assert buf[1024 + 30 * 32 + 7] == codec.fp8_quantize(v[7, 30], F32(2.0))


def _bf16(rng, *shape):
    return (rng.standard_normal(shape).astype(F32).view(np.uint32) >> 16).astype(np.uint16)


def test_kivi_cache_ring_and_pages():
    rng = np.random.default_rng(2)
    B, H, d, R, T = 2, 2, 32, 8, 77
    c = OracleCache(acc.KIVI, 2, 1, B, H, d, capacity=96, residual=R, in_dtype="bf16")
    k, v = _bf16(rng, B, T, H, d), _bf16(rng, B, T, H, d)
    c.append(0, k, v)
    q, n_r = acc.flush_plan(T, R)
    assert (q, n_r) == (64, 13)
    buf, mask = c.slab_image(0, 1, 1)
    ps = acc.page_bytes(acc.KIVI, d, 2)
    n_pages = acc.pages_per_slab(acc.KIVI, 96, R)
    assert n_pages == 2 and np.all(mask[:2 * ps] == 0xFF)
    ring0 = n_pages * ps
    row = d * 2
    for t in range(q, T):
        s = t % (R + 32)
        assert buf[ring0 + s * row: ring0 + (s + 1) * row].view(np.uint16).tolist() == \
            k[1, t, 1].tolist()
        vo = ring0 + (R + 32 + s) * row
        assert buf[vo:vo + row].view(np.uint16).tolist() == v[1, t, 1].tolist()
    assert mask[ring0:].sum() == 0xFF * 2 * n_r * row
    # page 1 holds tokens 32..63
    pb, _ = layout.kivi_page(bf16_bits_to_f32(k[1, 32:64, 1]), bf16_bits_to_f32(v[1, 32:64, 1]), 2)
    assert np.array_equal(buf[ps:2 * ps], pb)


def test_cache_chunking_independent():
    rng = np.random.default_rng(3)
    B, H, d = 1, 2, 32
    k, v = _bf16(rng, B, 100, H, d), _bf16(rng, B, 100, H, d)
    one = OracleCache(acc.KIVI, 4, 1, B, H, d, 128, residual=16)
    one.append(0, k, v)
    many = OracleCache(acc.KIVI, 4, 1, B, H, d, 128, residual=16)
    for a, b in [(0, 1), (1, 33), (33, 34), (34, 90), (90, 100)]:
        many.append(0, k[:, a:b], v[:, a:b])
    b1, m1 = one.cache_image()
    b2, m2 = many.cache_image()
    assert np.array_equal(m1, m2) and np.array_equal(b1 & m1, b2 & m2)


def test_cache_dequant_matches_pages():
    """dequantized() (used for attention) agrees with decoding the byte image."""
    rng = np.random.default_rng(4)
    B, H, d = 1, 1, 32
    k, v = _bf16(rng, B, 70, H, d), _bf16(rng, B, 70, H, d)
    c = OracleCache(acc.KIVI, 2, 1, B, H, d, 80, residual=4)
    c.append(0, k, v)
    kh, vh = c.dequantized(0)
    buf, _ = c.slab_image(0, 0, 0)
    ps = acc.page_bytes(acc.KIVI, d, 2)
    nb = 32 * d * 2 // 8
    for p in range(2):
        pg = buf[p * ps:(p + 1) * ps]
        kc = layout.unpack_fields(pg[:nb], 2, 32 * d).reshape(32, d)
        ks, kz = pg[nb:nb + 4 * d].view(F32), pg[nb + 4 * d:nb + 8 * d].view(F32)
        assert np.array_equal(kh[0, 0, p * 32:(p + 1) * 32], kc * ks.astype(np.float64) + kz)
    assert np.array_equal(kh[0, 0, 64:], bf16_bits_to_f32(k[0, 64:, 0]))   # ring exact
    assert np.array_equal(vh[0, 0, 64:], bf16_bits_to_f32(v[0, 64:, 0]))


def test_cache_decode_small():
    rng = np.random.default_rng(5)
    B, H, Hq, d = 2, 2, 4, 32
    c = OracleCache(acc.SYM_TOKEN, 8, 1, B, H, d, 64, in_dtype="f32")
    k = rng.standard_normal((B, 40, H, d)).astype(F32)
    v = rng.standard_normal((B, 40, H, d)).astype(F32)
    c.append(0, k, v)
    q = rng.standard_normal((B, Hq, d))
    out = c.decode(0, q)
    kh, vh = c.dequantized(0)
    # 8-bit symmetric is close to the unquantised attention
    from oracle import attention
    ref = attention.decode(q, np.transpose(k, (0, 2, 1, 3)), np.transpose(v, (0, 2, 1, 3)),
                           1 / np.sqrt(d))
    assert np.max(np.abs(out - ref)) < 0.02
    assert np.allclose(out[1, 2], attention.attend(q[1, 2], kh[1, 1], vh[1, 1], 1 / np.sqrt(d)))


def test_bf16_page_layout():
    """K rows then V cols, two bytes per value (low byte first); a partial page
    defines only its tokens."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((32, 64)).astype(F32)
    v = rng.standard_normal((32, 64)).astype(F32)
    buf, mask = layout.bf16_page(k, v, 5)
    assert buf.size == mask.size == acc.page_bytes(acc.BF16_CACHE, 64, 16) == 8192
    kc = buf[:4096].view("<u2").reshape(32, 64)
    vc = buf[4096:].view("<u2").reshape(64, 32)
    assert np.array_equal(kc[:5], codec.bf16_encode(k[:5]))
    assert np.array_equal(vc[:, :5], codec.bf16_encode(v[:5]).T)
    assert np.all(mask[:5 * 128] == 0xFF) and np.all(mask[5 * 128:4096] == 0)
    vm = mask[4096:].reshape(64, 64)
    assert np.all(vm[:, :10] == 0xFF) and np.all(vm[:, 10:] == 0)


def test_kivi_page_value_bits():
    """A page with value codes narrower than key codes is the key half of the
    key-width page followed by the value half of the value-width page (keys and
    values are grouped and rounded independently), and the whole-cache oracle
    dequantises values at their own width."""
    rng = np.random.default_rng(11)
    d = 64
    k = rng.standard_normal((32, d)).astype(F32)
    v = rng.standard_normal((32, d)).astype(F32)
    for kb, vb in ((4, 2), (8, 2), (8, 4)):
        mixed, mask = layout.kivi_page(k, v, kb, vb)
        wide, _ = layout.kivi_page(k, v, kb)
        narrow, _ = layout.kivi_page(k, v, vb)
        kpart = 32 * d * kb // 8 + 8 * d
        vpart = 32 * d * vb // 8 + 256
        assert mixed.size == kpart + vpart == acc.page_bytes(acc.KIVI, d, kb, vb)
        assert np.array_equal(mixed[:kpart], wide[:kpart])
        assert np.array_equal(mixed[kpart:], narrow[narrow.size - vpart:])
        assert np.all(mask == 0xFF)
    B, H = 1, 2
    kk, vv = _bf16(rng, B, 90, H, d), _bf16(rng, B, 90, H, d)
    c42 = OracleCache(acc.KIVI, 4, 1, B, H, d, 96, residual=8, v_bits=2)
    c44 = OracleCache(acc.KIVI, 4, 1, B, H, d, 96, residual=8)
    c22 = OracleCache(acc.KIVI, 2, 1, B, H, d, 96, residual=8)
    for c in (c42, c44, c22):
        c.append(0, kk, vv)
    k42, v42 = c42.dequantized(0)
    assert np.array_equal(k42, c44.dequantized(0)[0])
    assert np.array_equal(v42, c22.dequantized(0)[1])
    # at d 64: 2 pages of 1024 B key codes + 512 B key scales/offsets + 512 B value
    # codes + 256 B value scales/offsets, then the ring of 40 bf16 K and V rows
    assert c42.slab_size() == 2 * (1024 + 512 + 512 + 256) + 2 * 40 * d * 2


def test_pack_3bit_worked_example(golden):
    """3-bit fields straddle bytes; the hand-packed bytes of the fixture."""
    ex = golden("qb_worked_examples.json")["pack_3bit"]
    got = layout.pack_fields(np.array(ex["codes"]), 3)
    assert got.tolist() == ex["bytes"]
    assert layout.unpack_fields(got, 3, 8).tolist() == ex["codes"]


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_three_bit_page_sizes(d):
    """3-bit K rows and V cols: 12 d bytes each; a KIVI page stays a multiple
    of 256 bytes with both widths 3, and with 3 bits next to another width
    from d = 64 on (d = 32 then gives 128 bytes over: that combination is
    not supported)."""
    for kb, vb in ((3, 3), (4, 3), (8, 3), (3, 2)):
        n = acc.page_bytes(acc.KIVI, d, kb, vb)
        assert n == 32 * d * kb // 8 + 8 * d + 32 * d * vb // 8 + 256
        assert (n % 256 == 0) == (kb == vb or d >= 64)


@pytest.mark.parametrize("vb", [2, 3, 4, 8])
def test_fp8k_symv_page_halves(vb):
    """Keys and values in different cache types: the page is the FP8 page's key
    rows (one E4M3 byte per value, the key scale of the KV head) followed by
    the symmetric page's value columns and value scales; each half decoded
    here from the bytes by hand, with a partial page's undefined tokens masked."""
    rng = np.random.default_rng(11 + vb)
    d, n = 64, 29
    k = rng.standard_normal((32, d)).astype(F32) * 3
    v = rng.standard_normal((32, d)).astype(F32)
    ks = F32(0.0125)
    buf, mask = layout.fp8k_symv_page(k, v, ks, vb, n)
    assert buf.size == mask.size == acc.page_bytes(acc.FP8K_SYMV, d, 8, vb) == 32 * d + 32 * d * vb // 8 + 256
    assert buf.size % 256 == 0
    # key rows: byte (t, c) is the E4M3 code of k[t, c] / ks for t < n, undefined after
    kb = buf[:32 * d].reshape(32, d)
    assert np.array_equal(kb[:n], codec.fp8_quantize(k[:n], ks, "e4m3"))
    assert np.all(mask[:n * d] == 0xFF) and np.all(mask[n * d:32 * d] == 0)
    # value columns: channel c's 32 fields of vb bits (two's complement), then
    # one float32 scale per token
    vbytes = buf[32 * d:32 * d + 32 * d * vb // 8]
    f = layout.unpack_fields(vbytes, vb, 32 * d).reshape(d, 32).astype(np.int64)
    f = np.where(f >= 1 << (vb - 1), f - (1 << vb), f)
    vs = buf[32 * d + 32 * d * vb // 8:32 * d + 32 * d * vb // 8 + 128].view(F32)
    c, s = codec.sym_quantize(v, vb, axis=1)
    assert np.array_equal(f.T[:n], c[:n]) and np.array_equal(vs[:n], s[:n])
    sm = mask[32 * d + 32 * d * vb // 8:]
    assert np.all(vs[n:] == 0) and np.all(sm[:4 * n] == 0xFF) and np.all(sm[4 * n:] == 0)   # (padding: mask 0)
    # each value is within half a step of its code's value (symmetric rounding)
    assert np.all(np.abs(f.T[:n] * vs[:n, None].astype(np.float64) - v[:n]) <= vs[:n, None] / 2 + 1e-7)


def test_fp8k_symv_cache_dequant_matches_bytes():
    """dequantized() of a cache with FP8 keys and symmetric values equals the
    byte image decoded by hand (keys: code value x key scale; values: field x
    token scale), for tokens across several appends and a partial last page."""
    rng = np.random.default_rng(12)
    B, H, d, vb = 2, 2, 32, 4
    c = OracleCache(acc.FP8K_SYMV, 8, 1, B, H, d, 96, in_dtype="f32", v_bits=vb)
    scales = np.array([0.02, 0.05], F32)
    k = rng.standard_normal((B, 70, H, d)).astype(F32)
    v = rng.standard_normal((B, 70, H, d)).astype(F32)
    for a, z in ((0, 33), (33, 34), (34, 70)):
        c.append(0, k[:, a:z], v[:, a:z], k_scale=scales)
    kh, vh = c.dequantized(0)
    ps = acc.page_bytes(acc.FP8K_SYMV, d, 8, vb)
    for b in range(B):
        for h in range(H):
            buf, _ = c.slab_image(0, b, h)
            for p in range(3):
                n = min(32, 70 - 32 * p)
                pg = buf[p * ps:(p + 1) * ps]
                kc = pg[:32 * d].reshape(32, d)[:n]
                assert np.array_equal(kh[b, h, 32 * p:32 * p + n],
                                      codec.fp8_dequantize(kc, scales[h], "e4m3"))
                f = layout.unpack_fields(pg[32 * d:32 * d + 32 * d * vb // 8], vb, 32 * d)
                f = f.reshape(d, 32).astype(np.int64)
                f = np.where(f >= 8, f - 16, f).T[:n]
                sc = pg[32 * d + 32 * d * vb // 8:32 * d + 32 * d * vb // 8 + 128].view(F32)[:n]
                assert np.array_equal(vh[b, h, 32 * p:32 * p + n], f * sc[:, None].astype(np.float64))


@pytest.mark.parametrize("fmt_scheme,fmt", [(acc.FP8_E4M3, "e4m3"), (acc.FP8_E5M2, "e5m2")])
def test_fp8_cache_open_page_rows_then_columns(fmt_scheme, fmt):
    """dequantized() of an FP8 cache equals its byte image decoded by hand
    after every append of a sequence that opens, extends and closes pages
    (one token, a chunk ending inside a page, one closing it and opening the
    next): a full page's values are read as channel columns, the last page's
    (fewer than 32 tokens) as token rows."""
    rng = np.random.default_rng(21)
    B, H, d = 1, 2, 32
    c = OracleCache(fmt_scheme, 8, 1, B, H, d, 128, in_dtype="f32")
    ks, vs = np.array([0.02, 0.05], F32), np.array([0.03, 0.01], F32)
    k = rng.standard_normal((B, 100, H, d)).astype(F32)
    v = rng.standard_normal((B, 100, H, d)).astype(F32)
    ps = acc.page_bytes(fmt_scheme, d, 8)
    for a, z in ((0, 1), (1, 20), (20, 31), (31, 32), (32, 45), (45, 70), (70, 71), (71, 100)):
        c.append(0, k[:, a:z], v[:, a:z], k_scale=ks, v_scale=vs)
        kh, vh = c.dequantized(0)
        for h in range(H):
            buf, mask = c.slab_image(0, 0, h)
            for p in range(-(-z // 32)):
                n = min(32, z - 32 * p)
                pg = buf[p * ps:(p + 1) * ps]
                kc = pg[:32 * d].reshape(32, d)[:n]
                assert np.array_equal(kh[0, h, 32 * p:32 * p + n], codec.fp8_dequantize(kc, ks[h], fmt))
                vb = pg[32 * d:].reshape(32, d)
                vc = vb[:n] if n < 32 else vb.T            # open page: rows; full: columns
                assert np.array_equal(vh[0, h, 32 * p:32 * p + n], codec.fp8_dequantize(vc, vs[h], fmt))


@pytest.mark.parametrize("vb", [2, 3, 4, 8])
def test_fp8k_kiviv_page_halves(vb):
    """FP8 keys with KIVI values: the FP8 page's key rows, then value columns
    of unsigned vb-bit fields, then each token's fp32 scale and fp32 offset.
    Decoded here from the bytes by hand: each token's smallest value has code
    0 and decodes to itself, its largest has code 2^vb - 1, every value lies
    within half a step of its decoded value, and a partial page's undefined
    tokens are masked."""
    rng = np.random.default_rng(31 + vb)
    d, n = 64, 27
    k = rng.standard_normal((32, d)).astype(F32) * 3
    v = rng.standard_normal((32, d)).astype(F32) + F32(0.5)
    ks = F32(0.0125)
    buf, mask = layout.fp8k_kiviv_page(k, v, ks, vb, n)
    vend = 32 * d + 32 * d * vb // 8
    assert buf.size == mask.size == acc.page_bytes(acc.FP8K_KIVIV, d, 8, vb) == vend + 256
    assert buf.size % 256 == 0
    kb = buf[:32 * d].reshape(32, d)
    assert np.array_equal(kb[:n], codec.fp8_quantize(k[:n], ks, "e4m3"))
    assert np.all(mask[:n * d] == 0xFF) and np.all(mask[n * d:32 * d] == 0)
    f = layout.unpack_fields(buf[32 * d:vend], vb, 32 * d).reshape(d, 32).T.astype(np.int64)   # [token, channel]
    s = buf[vend:vend + 128].view(F32).astype(np.float64)
    z = buf[vend + 128:vend + 256].view(F32).astype(np.float64)
    L = (1 << vb) - 1
    for t in range(n):
        lo, hi = int(np.argmin(v[t])), int(np.argmax(v[t]))
        assert f[t, lo] == 0 and z[t] == v[t, lo] and f[t, hi] == L
        assert np.isclose(s[t], (float(v[t, hi]) - float(v[t, lo])) / L, rtol=1e-6)
        assert np.all(np.abs(f[t] * s[t] + z[t] - v[t]) <= s[t] / 2 * (1 + 1e-5) + 1e-7)
    vm = mask[32 * d:vend]
    assert np.array_equal(vm, np.tile(layout._valid_fields_mask(n, 32, vb), d))
    sm = mask[vend:]
    for part in (sm[:128], sm[128:]):
        assert np.all(part[:4 * n] == 0xFF) and np.all(part[4 * n:] == 0)


def test_fp8k_kiviv_cache_dequant_matches_bytes():
    """dequantized() of a cache with FP8 keys and KIVI values equals the byte
    image decoded by hand (keys: code value x key scale; values: field x token
    scale + token offset), across several appends and a partial last page."""
    rng = np.random.default_rng(13)
    B, H, d, vb = 2, 2, 32, 4
    c = OracleCache(acc.FP8K_KIVIV, 8, 1, B, H, d, 96, in_dtype="f32", v_bits=vb)
    scales = np.array([0.02, 0.05], F32)
    k = rng.standard_normal((B, 70, H, d)).astype(F32)
    v = rng.standard_normal((B, 70, H, d)).astype(F32)
    for a, z in ((0, 1), (1, 33), (33, 70)):
        c.append(0, k[:, a:z], v[:, a:z], k_scale=scales)
    kh, vh = c.dequantized(0)
    ps = acc.page_bytes(acc.FP8K_KIVIV, d, 8, vb)
    vend = 32 * d + 32 * d * vb // 8
    for b in range(B):
        for h in range(H):
            buf, _ = c.slab_image(0, b, h)
            for p in range(3):
                n = min(32, 70 - 32 * p)
                pg = buf[p * ps:(p + 1) * ps]
                kc = pg[:32 * d].reshape(32, d)[:n]
                assert np.array_equal(kh[b, h, 32 * p:32 * p + n],
                                      codec.fp8_dequantize(kc, scales[h], "e4m3"))
                f = layout.unpack_fields(pg[32 * d:vend], vb, 32 * d).reshape(d, 32).T[:n]
                sc = pg[vend:vend + 128].view(F32)[:n].astype(np.float64)
                zz = pg[vend + 128:vend + 256].view(F32)[:n].astype(np.float64)
                assert np.array_equal(vh[b, h, 32 * p:32 * p + n], f * sc[:, None] + zz[:, None])
