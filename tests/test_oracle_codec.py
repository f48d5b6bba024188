"""Pins of oracle.codec: worked examples, invariants, brute force, a library routine."""

import numpy as np
import pytest
import torch

from oracle import codec

F32 = np.float32


# ---- KIVI Q_b --------------------------------------------------------------

def test_kivi_worked_examples(golden):
    for ex in golden("qb_worked_examples.json")["kivi"]:
        x = np.array(ex["x"], F32)
        codes, s, z = codec.kivi_quantize(x, ex["bits"], axis=0)
        assert codes.tolist() == ex["codes"], ex["name"]
        assert float(z) == ex["min"], ex["name"]
        if "scale" in ex:
            assert float(s) == ex["scale"], ex["name"]


def test_kivi_axes(golden):
    ex = golden("qb_worked_examples.json")["kivi_axes"]
    x = np.array(ex["x"], F32)
    c, s, z = codec.kivi_quantize(x, ex["bits"], axis=0)          # keys: per channel
    assert c.tolist() == ex["per_channel"]["codes"]
    assert s.tolist() == ex["per_channel"]["scale"]
    assert z.tolist() == ex["per_channel"]["min"]
    c, s, z = codec.kivi_quantize(x, ex["bits"], axis=1)          # values: per token
    assert c.tolist() == ex["per_token_codes"]
    assert z.tolist() == ex["per_token_min"]


def _groups(seed, n_groups, g, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_groups, g)).astype(F32) * F32(scale)
    return x


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_kivi_error_bound_and_extremes(bits):
    x = _groups(bits, 4000, 32)
    x[::7] *= F32(1000.0)
    x[1::11] *= F32(1e-30)                     # tiny (subnormal-range) groups
    codes, s, z = codec.kivi_quantize(x, bits, axis=1)
    L = 2 ** bits - 1
    xh = codec.kivi_dequantize(codes, s, z, axis=1)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(x.astype(np.float64) - xh)
    # |x - x^| <= s/2, with slack for the float32 rounding of s and of (x-min)/s
    assert np.all(err <= s64 / 2 + s64 * L * 2.0 ** -21 + 1e-45)
    assert codes.max() <= L
    amin = x.argmin(axis=1)
    amax = x.argmax(axis=1)
    rows = np.arange(len(x))
    assert np.all(codes[rows, amin] == 0)
    assert np.all(xh[rows, amin] == x[rows, amin])            # min decodes exactly
    assert np.all(codes[rows, amax] == L)
    assert np.all(z == x.min(axis=1))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_kivi_bruteforce_nearest_level(bits):
    """Code = the nearest of the 2^b levels k*s + z, except inside a tiny band
    around exact midpoints where float32 rounding of (x-z)/s decides."""
    x = _groups(10 + bits, 300, 8)
    codes, s, z = codec.kivi_quantize(x, bits, axis=1)
    for i in range(len(x)):
        si, zi = float(s[i]), float(z[i])
        for j in range(x.shape[1]):
            xv = float(x[i, j])
            dists = [abs(xv - (k * si + zi)) for k in range(2 ** bits)]
            best = int(np.argmin(dists))
            u = (xv - zi) / si
            near_tie = abs(u - np.floor(u) - 0.5) < 2.0 ** -20
            assert codes[i, j] == best or near_tie


def test_kivi_signed_zero_min():
    x = np.array([[-0.0, 1.0, 2.0, 3.0]], F32)
    _, s, z = codec.kivi_quantize(x, 2, axis=1)
    assert not np.signbit(z[0]) and z[0] == 0.0


def test_per_channel_beats_per_token_on_outlier_channels():
    """Qualitative claim of 'Keys and values are shaped differently': with a few
    large channels in every token, per-channel 2-bit grouping loses less than
    per-token. (The page's own 48%/16% slice is not published: parity unpinned
    for the numbers themselves.)"""
    rng = np.random.default_rng(0)
    K = rng.standard_normal((32 * 64, 128)).astype(F32)
    K[:, [3, 50, 77, 120]] *= F32(20.0)
    Kg = K.reshape(64, 32, 128)
    c, s, z = codec.kivi_quantize(Kg, 2, axis=1)                  # per channel
    e_ch = np.linalg.norm(codec.kivi_dequantize(c, s, z, axis=1) - Kg) / np.linalg.norm(Kg)
    c, s, z = codec.kivi_quantize(Kg, 2, axis=2)                  # per token
    e_tok = np.linalg.norm(codec.kivi_dequantize(c, s, z, axis=2) - Kg) / np.linalg.norm(Kg)
    assert e_ch < e_tok


# ---- symmetric -------------------------------------------------------------

def test_sym_worked_examples(golden):
    for ex in golden("qb_worked_examples.json")["sym"]:
        x = np.array(ex["x"], F32)
        codes, s = codec.sym_quantize(x, ex["bits"], axis=0)
        assert codes.tolist() == ex["codes"], ex["name"]
        assert float(s) == ex["scale"], ex["name"]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_sym_invariants(bits):
    x = _groups(20 + bits, 3000, 32)
    x[::5] *= F32(300.0)
    codes, s = codec.sym_quantize(x, bits, axis=1)
    Q = 2 ** (bits - 1) - 1
    xh = codec.sym_dequantize(codes, s, axis=1)
    s64 = s.astype(np.float64)[:, None]
    assert np.all(np.abs(x - xh) <= s64 / 2 + s64 * Q * 2.0 ** -21)
    rows = np.arange(len(x))
    am = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[rows, am]) == Q)
    assert np.all(np.sign(codes[rows, am]) == np.sign(x[rows, am]))
    assert codes.min() >= -Q and codes.max() <= Q
    z, zs = codec.sym_quantize(np.zeros((2, 8), F32), bits, axis=1)
    assert np.all(z == 0) and np.all(zs == 0)


# ---- FP8 E4M3 --------------------------------------------------------------

def test_e4m3_table_definition():
    t = codec.E4M3_TABLE
    assert t[0x7E] == 448.0 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0)                      # codes increase with value
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])   # sign bit


def test_e4m3_worked_examples(golden):
    cases = golden("qb_worked_examples.json")["e4m3"]["cases"]
    y = np.array([c[0] for c in cases], F32)
    want = np.array([c[1] for c in cases], np.uint8)
    assert codec.e4m3_encode(y).tolist() == want.tolist()
    assert codec.e4m3_encode_bruteforce(y).tolist() == want.tolist()


def test_e4m3_vectorised_equals_bruteforce():
    rng = np.random.default_rng(5)
    y = np.concatenate([
        rng.standard_normal(3000).astype(F32) * F32(100),
        (rng.standard_normal(1000) * 0.01).astype(F32),
        # every midpoint between adjacent finite values, and its neighbours
        ((codec.E4M3_TABLE[:0x7E] + codec.E4M3_TABLE[1:0x7F]) / 2).astype(F32),
    ])
    mids = ((codec.E4M3_TABLE[:0x7E] + codec.E4M3_TABLE[1:0x7F]) / 2).astype(F32)
    y = np.concatenate([y, np.nextafter(mids, F32(0)), np.nextafter(mids, F32(1e6)), -y])
    assert np.array_equal(codec.e4m3_encode(y), codec.e4m3_encode_bruteforce(y))


def test_e4m3_matches_torch_in_range():
    """torch.float8_e4m3fn rounds to nearest-even; it agrees wherever |y| < 464
    (above that torch returns NaN while this reading saturates)."""
    rng = np.random.default_rng(6)
    y = np.concatenate([rng.uniform(-463.9, 463.9, 20000), rng.standard_normal(20000),
                        rng.standard_normal(5000) * 1e-3]).astype(F32)
    ours = codec.e4m3_encode(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_relative_error():
    rng = np.random.default_rng(7)
    y = rng.uniform(2.0 ** -6, 448.0, 20000).astype(F32)
    back = codec.e4m3_decode(codec.e4m3_encode(y))
    assert np.all(np.abs(back - y) / y <= 2.0 ** -4)
    big = np.array([449.0, 1e4, -3e38, 1e30], F32)
    assert np.array_equal(np.abs(codec.e4m3_decode(codec.e4m3_encode(big))), [448.0] * 4)


def test_fp8_quantize_uses_scale():
    x = np.array([2.0, -4.0, 896.0, 1000.0], F32)
    c = codec.fp8_quantize(x, F32(2.0))
    assert codec.fp8_dequantize(c, 2.0).tolist() == [2.0, -4.0, 896.0, 896.0]


# ---- bfloat16 (the unquantised 16-bit baseline) ------------------------------

def test_bf16_matches_torch():
    """torch's float32 -> bfloat16 conversion rounds to nearest, ties to even."""
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 0x7F800000, 20000, dtype=np.uint32)       # finite positives
    bits = np.concatenate([bits, bits | 0x80000000,
                           (bits & 0xFFFF0000) | 0x8000,              # exact ties
                           (bits & 0xFFFF0000) | 0x7FFF, (bits & 0xFFFF0000) | 0x8001])
    x = bits.view(F32)
    x = x[np.abs(x) < np.float32(3.0e38)]          # stay clear of rounding up to infinity
    ours = codec.bf16_encode(x)
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_nearest_by_brute_force():
    """For each input, no other bfloat16 pattern near it is closer, and ties
    pick the even pattern (fp64 distances, small inputs)."""
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(300), [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0,
                                                   2.0 ** -130, 65504.0]]).astype(F32)
    codes = codec.bf16_encode(x).astype(np.int64)
    for xi, c in zip(x, codes):
        best = codec.bf16_decode(np.uint16(c))
        for cand in (c - 2, c - 1, c + 1, c + 2):
            if 0 <= cand <= 0xFFFF and (cand & 0x7F80) != 0x7F80 and (cand >> 15) == (c >> 15):
                dc, db = abs(codec.bf16_decode(np.uint16(cand)) - float(xi)), abs(best - float(xi))
                assert dc > db or (dc == db and c % 2 == 0), (xi, c, cand)


def test_bf16_inputs_are_kept():
    raw = np.array([0x3F80, 0xC049, 0x0001, 0x8000, 0x7F7F], np.uint16)
    x = (raw.astype(np.uint32) << 16).view(F32)
    assert np.array_equal(codec.bf16_encode(x), raw)
    assert codec.bf16_decode(raw).tolist() == x.astype(np.float64).tolist()


# ---- FP8 E5M2 -------------------------------------------------------------------

def test_e5m2_table_definition():
    assert codec.e5m2_value(0x3C) == 1.0 and codec.e5m2_value(0xBC) == -1.0
    assert codec.e5m2_value(0x7B) == 57344.0                 # largest finite
    assert codec.e5m2_value(0x04) == 2.0 ** -14              # smallest normal
    assert codec.e5m2_value(0x01) == 2.0 ** -16              # smallest subnormal
    assert codec.e5m2_value(0x7C) == float("inf") and np.isnan(codec.e5m2_value(0x7D))
    mags = codec.E5M2_TABLE[:0x7C]
    assert np.all(np.diff(mags) > 0)                          # increasing with the code


def test_e5m2_vectorised_equals_bruteforce():
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.standard_normal(400) * 10.0 ** rng.integers(-6, 5, 400),
                        [0.0, -0.0, 57344.0, 60000.0, 1e9, 2.0 ** -17, 3 * 2.0 ** -17,
                         1.125, 1.375, -1.625]]).astype(F32)
    assert np.array_equal(codec.e5m2_encode(y), codec.e5m2_encode_bruteforce(y))


def test_e5m2_matches_torch_in_range():
    """torch.float8_e5m2 rounds to nearest-even and overflows to infinity; it
    agrees wherever |y| < 61440 (the midpoint above 57344)."""
    rng = np.random.default_rng(12)
    y = np.concatenate([rng.uniform(-61439.0, 61439.0, 20000), rng.standard_normal(20000),
                        rng.standard_normal(5000) * 1e-5]).astype(F32)
    ours = codec.e5m2_encode(y)
    theirs = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e5m2_saturates_and_scales():
    big = np.array([57344.0, 61440.0, 1e30, -7e4], F32)
    assert np.array_equal(np.abs(codec.e5m2_decode(codec.e5m2_encode(big))), [57344.0] * 4)
    rng = np.random.default_rng(13)
    y = rng.uniform(2.0 ** -14, 57344.0, 20000).astype(F32)
    back = codec.e5m2_decode(codec.e5m2_encode(y))
    assert np.all(np.abs(back - y) / y <= 2.0 ** -3)          # half of a 2-bit mantissa step
    # 1e5 / 2 = 50000 lies between 49152 and 57344, nearer the first;
    # 1.2e5 / 2 = 60000 is beyond the largest finite value and saturates
    x = np.array([2.0, -4.0, 1.0e5, 1.2e5], F32)
    c = codec.fp8_quantize(x, F32(2.0), "e5m2")
    assert codec.fp8_dequantize(c, 2.0, "e5m2").tolist() == [2.0, -4.0, 98304.0, 114688.0]
