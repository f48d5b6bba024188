"""Pins of the oracle's paged-cache byte image (oracle.cache.paged_image).

A paged cache only moves pages: the pins read the image back through the
block table, independently of how it was written -- field by field with the
layout decoders -- and compare with the oracle's dequantised cache, and check
that a permuted table moves every page and ring without changing a byte of it.
(KIVI page, Key points: KIVI pairs with PagedAttention.)"""

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import layout
from oracle.cache import OracleCache, RaggedCache, paged_image

B, H, D, CAP, R = 3, 2, 32, 200, 16


def filled(scheme, bits, lens, seed=0):
    rng = np.random.default_rng(seed)
    rc = RaggedCache(scheme, bits, 2, B, H, D, CAP, residual=R if scheme == acc.KIVI else 0,
                     in_dtype="f32")
    for layer in range(2):
        for b, n in enumerate(lens):
            k = rng.standard_normal((n, H, D)).astype(np.float32)
            v = rng.standard_normal((n, H, D)).astype(np.float32)
            ks = vs = None
            if scheme == acc.FP8_E4M3:
                ks = vs = np.full(H, 0.02, np.float32)
            rc.append(layer, b, k, v, ks, vs)
    return rc


def tables(P, nb, seed):
    ident = np.arange(B * P, dtype=np.int32).reshape(B, P)
    perm = np.random.default_rng(seed).permutation(nb)[:B * P].astype(np.int32).reshape(B, P)
    return ident, perm


@pytest.mark.parametrize("scheme,bits", [(acc.KIVI, 2), (acc.KIVI, 4), (acc.FP8_E4M3, 8)])
def test_pages_read_back_through_the_table(scheme, bits):
    lens = [200, 77, 140]
    rc = filled(scheme, bits, lens)
    one = rc.seqs[0]
    P = acc.pages_per_slab(scheme, CAP, one.residual)
    nb = B * P + 5
    ps = one.page_size()
    rb = acc.ring_bytes(scheme, D, one.residual, 4)
    ring_region = -(-(2 * B * H * rb) // 256) * 256
    ident, perm = tables(P, nb, 7)
    for table in (ident, perm):
        buf, mask = paged_image(rc, table, nb)
        assert buf.size == ring_region + 2 * nb * H * ps
        for layer in range(2):
            for b in range(B):
                kh, vh = rc.seqs[b].dequantized(layer)
                T = lens[b]
                q = acc.flush_plan(T, one.residual)[0] if scheme == acc.KIVI else T
                for p in range((q + 31) // 32):
                    for h in range(H):
                        o = ring_region + ((layer * nb + int(table[b, p])) * H + h) * ps
                        page = buf[o:o + ps]
                        n = min(32, q - 32 * p)
                        if scheme == acc.KIVI:
                            codes = layout.unpack_fields(page[:32 * D * bits // 8], bits, 32 * D)
                            s = page[32 * D * bits // 8:32 * D * bits // 8 + 4 * D].view(np.float32)
                            z = page[32 * D * bits // 8 + 4 * D:32 * D * bits // 8 + 8 * D].view(np.float32)
                            k = codes.reshape(32, D) * s.astype(np.float64) + z.astype(np.float64)
                            assert np.array_equal(k, kh[0, h, 32 * p:32 * p + 32])
                        else:
                            from oracle import codec
                            e = codec.e4m3_decode(page[:32 * D].reshape(32, D)[:n]) * np.float64(np.float32(0.02))
                            assert np.array_equal(e, kh[0, h, 32 * p:32 * p + n])
                if scheme == acc.KIVI:   # the ring rows, exact, in slot t mod (R + 32)
                    for h in range(H):
                        o = ((layer * B + b) * H + h) * rb
                        rows = buf[o:o + rb].view(np.float32).reshape(2, R + 32, D)
                        for t in range(q, T):
                            assert np.array_equal(rows[0, t % (R + 32)], kh[0, h, t])
                            assert np.array_equal(rows[1, t % (R + 32)], vh[0, h, t])


def test_permuted_table_moves_pages_unchanged():
    lens = [200, 150, 33]
    rc = filled(acc.KIVI, 2, lens, seed=3)
    one = rc.seqs[0]
    P = acc.pages_per_slab(acc.KIVI, CAP, R)
    nb = B * P + 3
    ident, perm = tables(P, nb, 11)
    bi, mi = paged_image(rc, ident, nb)
    bp, mp = paged_image(rc, perm, nb)
    assert not np.array_equal(bi, bp)
    ps = one.page_size()
    ring_region = -(-(2 * B * H * acc.ring_bytes(acc.KIVI, D, R, 4)) // 256) * 256
    assert np.array_equal(bi[:ring_region], bp[:ring_region])
    for layer in range(2):
        for b in range(B):
            for p in range(P):
                for h in range(H):
                    oi = ring_region + ((layer * nb + int(ident[b, p])) * H + h) * ps
                    op = ring_region + ((layer * nb + int(perm[b, p])) * H + h) * ps
                    assert np.array_equal(bi[oi:oi + ps], bp[op:op + ps])
                    assert np.array_equal(mi[oi:oi + ps], mp[op:op + ps])
