"""Pins of the oracle's dense-and-sparse KIVI encoding (codec.kivi_quantize_sparse,
its page layout and cache decode).

The pages say only that KVQuant moves a small fraction of outliers, per vector,
into a separate sparse representation (KVQuant page, Summary; "Quantizing the
KV cache", going deeper: a few outliers kept in a sparse side matrix). The
reading pinned here: each quantisation vector (a key channel's 32 tokens of one
page, a value token's channels) moves its largest-magnitude value, stored
exactly with its index, and the rest is rounded by Q_b over its own range."""

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import attention, codec, layout
from oracle.cache import OracleCache

F32 = np.float32


def test_worked_examples(golden):
    g = golden("sparse_worked_examples.json")
    for case in g["cases"]:
        x = np.array(case["x"], F32)
        c, s, z, ov, oi = codec.kivi_quantize_sparse(x, case["bits"], axis=0)
        assert int(oi[0]) == case["out_index"], case["name"]
        assert float(ov[0]) == case["out_value"], case["name"]
        assert float(z) == case["min"], case["name"]
        assert float(s) == case["scale"], case["name"]
        assert c.tolist() == case["codes"], case["name"]
        xh = codec.kivi_dequantize_sparse(c, s, z, ov, oi, axis=0)
        assert xh[case["out_index"]] == case["out_value"]     # the outlier comes back exactly


def _vectors(seed, shape, spikes=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(F32)
    if spikes:   # a planted spike in some vectors, others plain
        m = rng.random(shape) < 0.01
        x = np.where(m, x * F32(60.0), x)
    return x


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("axis", [0, 1])
def test_invariants(bits, axis):
    x = _vectors(bits * 10 + axis, (32, 64))
    c, s, z, ov, oi = codec.kivi_quantize_sparse(x, bits, axis=axis)
    L = 2 ** bits - 1
    xm = np.moveaxis(x, axis, -1)
    cm = np.moveaxis(c, axis, -1)
    n = xm.shape[-1]
    for v in range(xm.shape[0]):
        i = int(oi[v, 0])
        # the moved value is a largest magnitude, the first such index
        mags = np.abs(xm[v])
        assert mags[i] == mags.max() and np.all(mags[:i] < mags[i])
        assert ov[v, 0] == xm[v, i]
        assert cm[v, i] == 0
        rest = np.delete(xm[v], i)
        # the dense part is exactly the plain quantiser over the remaining values
        c2, s2, z2 = codec.kivi_quantize(rest, bits, axis=0)
        assert s[v] == s2 and z[v] == z2
        assert np.array_equal(np.delete(cm[v], i), c2)
        assert np.all(cm[v] <= L)
        # half a step away at most, and never a coarser step than without the move
        sp = codec.kivi_quantize(xm[v], bits, axis=0)[1]
        assert s[v] <= sp
    xh = codec.kivi_dequantize_sparse(c, s, z, ov, oi, axis=axis)
    xhm = np.moveaxis(xh, axis, -1)
    for v in range(xm.shape[0]):
        i = int(oi[v, 0])
        assert xhm[v, i] == float(xm[v, i])                  # exact
        err = np.abs(np.delete(xhm[v], i) - np.delete(xm[v], i).astype(np.float64))
        assert np.all(err <= float(s[v]) / 2 + float(s[v]) * L * 2.0 ** -22 + 1e-30)


def test_selection_bruteforce():
    """Python loops pick the outlier on tiny vectors, including exact ties in
    magnitude (+a and -a), zeros and -0."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        n = int(rng.integers(2, 9))
        x = rng.integers(-4, 5, n).astype(F32)
        if trial % 7 == 0:
            x[:] = -0.0
        c, s, z, ov, oi = codec.kivi_quantize_sparse(x, 2, axis=0)
        best = 0
        for j in range(1, n):
            if abs(float(x[j])) > abs(float(x[best])):
                best = j
        assert int(oi[0]) == best, (x, oi)


def test_spike_shrinks_the_error_of_the_others():
    """With a planted spike, moving it leaves the other values a finer grid."""
    x = _vectors(3, (32, 128), spikes=False)
    x[5, 7] = F32(300.0)
    plain = codec.kivi_dequantize(*codec.kivi_quantize(x, 2, axis=0), axis=0)
    sp = codec.kivi_dequantize_sparse(*codec.kivi_quantize_sparse(x, 2, axis=0), axis=0)
    col = np.abs(plain[:, 7] - x[:, 7])
    cols = np.abs(sp[:, 7] - x[:, 7])
    assert cols.max() < col.max() / 4      # about 0.7 against 4.3 here


def test_page_layout_side_matrix():
    """Byte positions of the side matrix (d = 128): after the dense page,
    key outliers [d] f32, value outliers [32] f32, key outlier tokens [d] u8,
    value outlier channels [32] u8, padded to a multiple of 256."""
    d = 128
    k = _vectors(8, (32, d))
    v = _vectors(9, (32, d))
    buf, mask = layout.kivi_page(k, v, 2, None, outliers=1)
    base = acc.page_bytes(acc.KIVI, d, 2)
    assert base == 3328 and buf.size == acc.page_bytes(acc.KIVI, d, 2, outliers=1) == 3328 + 1024
    assert buf.size % 256 == 0
    assert mask[:base + 5 * d + 160].all() and not mask[base + 5 * d + 160:].any()
    kc, ks, kz, ko, ki = codec.kivi_quantize_sparse(k, 2, axis=0)
    vc, vs, vz, vo, vi = codec.kivi_quantize_sparse(v, 2, axis=1)
    o = base
    assert np.array_equal(buf[o:o + 4 * d].view(F32), ko[:, 0]); o += 4 * d
    assert np.array_equal(buf[o:o + 128].view(F32), vo[:, 0]); o += 128
    assert np.array_equal(buf[o:o + d], ki[:, 0]); o += d
    assert np.array_equal(buf[o:o + 32], vi[:, 0])
    # key outlier of channel c is token ki[c] of that channel, exactly
    for c in (0, 17, 127):
        assert buf[base + 4 * c:base + 4 * c + 4].view(F32)[0] == k[ki[c, 0], c]
    # dense page: code 0 in the moved fields
    codes = layout.unpack_fields(buf[:32 * d * 2 // 8], 2, 32 * d).reshape(32, d)
    assert all(codes[ki[c, 0], c] == 0 for c in range(d))


@pytest.mark.parametrize("bits,v_bits,R,T", [(2, None, 8, 150), (4, 2, 0, 96), (3, 3, 16, 120)])
def test_decode_is_bruteforce_over_dense_plus_sparse(bits, v_bits, R, T):
    """Decode of a dense-and-sparse cache = textbook attention over rows built
    by hand: per page and vector, the plain quantiser's decoding of the other
    values, the outlier put back exactly; ring rows exact."""
    B, H, HQ, D = 2, 2, 4, 16
    rng = np.random.default_rng(bits + T)
    k = _vectors(rng.integers(1 << 30), (B, T, H, D))
    v = _vectors(rng.integers(1 << 30), (B, T, H, D))
    c = OracleCache(acc.KIVI, bits, 1, B, H, D, T, residual=R, in_dtype="f32", v_bits=v_bits,
                    outliers=1)
    c.append(0, k, v)
    q = rng.standard_normal((B, HQ, D)).astype(F32)
    got = c.decode(0, q)
    vb = bits if v_bits is None else v_bits
    qn, _ = acc.flush_plan(T, R)
    sm = 1.0 / np.sqrt(D)
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h].astype(np.float64).copy()
            vh = v[b, :, h].astype(np.float64).copy()
            for p in range(qn // 32):
                for ch in range(D):              # keys: per channel over the page's tokens
                    col = k[b, 32 * p:32 * p + 32, h, ch]
                    i = int(np.argmax(np.abs(col)))
                    rest = np.delete(col, i)
                    cc, s, z = codec.kivi_quantize(rest, bits, axis=0)
                    deq = list(cc.astype(np.float64) * float(s) + float(z))
                    deq.insert(i, float(col[i]))
                    kh[32 * p:32 * p + 32, ch] = deq
                for t in range(32 * p, 32 * p + 32):  # values: per token over the channels
                    row = v[b, t, h]
                    i = int(np.argmax(np.abs(row)))
                    cc, s, z = codec.kivi_quantize(np.delete(row, i), vb, axis=0)
                    deq = list(cc.astype(np.float64) * float(s) + float(z))
                    deq.insert(i, float(row[i]))
                    vh[t] = deq
            for g in range(HQ // H):
                hq = h * (HQ // H) + g
                want = attention.attend_bruteforce(q[b, hq].astype(np.float64), kh, vh, sm)
                assert np.max(np.abs(got[b, hq] - want)) < 1e-12
