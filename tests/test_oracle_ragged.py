"""Pins of the oracle's ragged-batch decode (per-sequence token counts).

A sequence of a ragged batch attends to its own first T_b tokens with its query
at position T_b - 1. The pins tie that to things fixed independently of the
ragged code path: the uniform decode (all T_b = T), a cache that only ever held
the first T_b tokens (for schemes whose encoding of a token never depends on
later tokens), and brute-force attention over the dequantised rows.
"""

import numpy as np
import pytest

from oracle import accounting as acc
from oracle import attention, rope
from oracle.cache import OracleCache

B, H, HQ, D = 3, 2, 4, 16


def filled(scheme, bits, T, residual=0, seed=0, rope_theta=0.0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    c = OracleCache(scheme, bits, 1, B, H, D, T, residual=residual, in_dtype="f32")
    ks = vs = None
    if scheme in (acc.FP8_E4M3, acc.FP8_E5M2):
        ks = (np.abs(k).max(axis=(0, 1, 3)) / 448.0).astype(np.float32)
        vs = (np.abs(v).max(axis=(0, 1, 3)) / 448.0).astype(np.float32)
    c.append(0, k, v, ks, vs)
    q = rng.standard_normal((B, HQ, D)).astype(np.float32)
    return c, k, v, ks, vs, q


@pytest.mark.parametrize("scheme,bits,R", [(acc.KIVI, 2, 16), (acc.SYM_TOKEN, 4, 0),
                                           (acc.FP8_E4M3, 8, 0), (acc.BF16_CACHE, 16, 0)])
def test_full_lengths_equal_uniform_decode(scheme, bits, R):
    c, *_, q = filled(scheme, bits, 90, residual=R)
    for theta in (0.0, 10000.0):
        want = c.decode(0, q, rope_theta=theta)
        got = c.decode(0, q, rope_theta=theta, seq_tokens=[90] * B)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("scheme,bits", [(acc.SYM_TOKEN, 4), (acc.SYM_TOKEN, 2), (acc.FP8_E4M3, 8),
                                         (acc.FP8_E5M2, 8), (acc.BF16_CACHE, 16)])
@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_prefix_equals_shorter_cache(scheme, bits, theta):
    """Per-token schemes encode a token independently of later ones, so
    sequence b of a ragged batch decodes exactly as a cache that only ever
    held its first T_b tokens (same query, position T_b - 1)."""
    T = 77
    c, k, v, ks, vs, q = filled(scheme, bits, T, seed=3)
    lens = [1, 40, 77]
    got = c.decode(0, q, rope_theta=theta, seq_tokens=lens)
    for b, Tb in enumerate(lens):
        short = OracleCache(scheme, bits, 1, B, H, D, Tb, in_dtype="f32")
        short.append(0, k[:, :Tb], v[:, :Tb], ks, vs)
        want = short.decode(0, q, rope_theta=theta)
        assert np.array_equal(got[b], want[b]), (b, Tb)


def test_kivi_prefix_is_bruteforce_over_dequantised_rows():
    """KIVI: the flush plan follows the fill level T, so a shorter sequence
    reads pages and ring rows of the full cache; the result is brute-force
    attention over those dequantised rows (tokens in a partial page, tokens in
    the ring, and the first token alone)."""
    T, R = 100, 8                       # q(T) = 64: two pages, 36 ring tokens
    c, *_, q = filled(acc.KIVI, 2, T, residual=R, seed=5)
    kh, vh = c.dequantized(0)
    lens = [1, 47, 83]                  # inside page 0, inside page 1, in the ring
    sm = 1.0 / np.sqrt(D)
    for theta in (0.0, 10000.0):
        got = c.decode(0, q, rope_theta=theta, seq_tokens=lens)
        for b, Tb in enumerate(lens):
            for h in range(HQ):
                g = attention.gqa_kv_head(h, HQ, H)
                kk = kh[b, g, :Tb]
                qq = q[b, h].astype(np.float64)
                if theta > 0:
                    kk = rope.rotate(kk, np.arange(Tb), theta)
                    qq = rope.rotate(qq, np.array(Tb - 1), theta)
                want = attention.attend_bruteforce(qq, kk, vh[b, g, :Tb], sm)
                np.testing.assert_allclose(got[b, h], want, rtol=0, atol=1e-12)


def test_kivi_short_sequence_reads_quantised_rows():
    """A sequence shorter than q(T) reads dequantised (not exact) rows: its
    result differs from a cache that held only its tokens in full precision
    (the ring of a short cache), which a plausible slip -- truncating before
    quantising -- would produce."""
    T, R = 100, 8
    c, k, v, ks, vs, q = filled(acc.KIVI, 2, T, residual=R, seed=7)
    Tb = 40
    got = c.decode(0, q, seq_tokens=[Tb] * B)
    short = OracleCache(acc.KIVI, 2, 1, B, H, D, Tb, residual=64, in_dtype="f32")   # all in the ring
    short.append(0, k[:, :Tb], v[:, :Tb])
    assert np.max(np.abs(got - short.decode(0, q))) > 1e-3


# ---- a ragged batch built by per-sequence appends (own fill levels) ----------

from oracle.cache import RaggedCache  # noqa: E402


def _history(scheme, T, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    ks = vs = None
    if scheme in (acc.FP8_E4M3, acc.FP8_E5M2):
        ks = (np.abs(k).max(axis=(0, 1, 3)) / 448.0).astype(np.float32)
        vs = (np.abs(v).max(axis=(0, 1, 3)) / 448.0).astype(np.float32)
    return k, v, ks, vs


@pytest.mark.parametrize("scheme,bits,R", [(acc.KIVI, 2, 16), (acc.KIVI, 4, 0), (acc.SYM_TOKEN, 4, 0),
                                           (acc.FP8_E4M3, 8, 0), (acc.BF16_CACHE, 16, 0)])
def test_ragged_equal_appends_equal_batch_cache(scheme, bits, R):
    """Every sequence appending the same chunks gives the batch cache's bytes,
    mask and decode, bit for bit."""
    T = 130
    k, v, ks, vs = _history(scheme, T, 11)
    batch = OracleCache(scheme, bits, 1, B, H, D, 160, residual=R, in_dtype="f32")
    rag = RaggedCache(scheme, bits, 1, B, H, D, 160, residual=R, in_dtype="f32")
    t = 0
    for n in (50, 1, 0, 79):
        if n:
            batch.append(0, k[:, t:t + n], v[:, t:t + n], ks, vs)
        for b in range(B):
            rag.append(0, b, k[b, t:t + n], v[b, t:t + n], ks, vs)
        t += n
    bb, bm = batch.cache_image()
    rb, rm = rag.cache_image()
    assert np.array_equal(bb, rb) and np.array_equal(bm, rm)
    q = np.random.default_rng(2).standard_normal((B, HQ, D)).astype(np.float32)
    for theta in (0.0, 10000.0):
        assert np.array_equal(rag.decode(0, q, rope_theta=theta), batch.decode(0, q, rope_theta=theta))


@pytest.mark.parametrize("scheme,bits", [(acc.SYM_TOKEN, 2), (acc.FP8_E5M2, 8), (acc.BF16_CACHE, 16)])
def test_ragged_fill_equals_masked_prefix_for_per_token_schemes(scheme, bits):
    """Per-token schemes: sequences filled to different lengths decode as the
    prefixes of a cache filled to the longest (two independent
    constructions: per-sequence caches vs one batch cache read in part)."""
    T = 90
    k, v, ks, vs = _history(scheme, T, 13)
    lens = [5, 90, 33]
    full = OracleCache(scheme, bits, 1, B, H, D, T, in_dtype="f32")
    full.append(0, k, v, ks, vs)
    rag = RaggedCache(scheme, bits, 1, B, H, D, T, in_dtype="f32")
    for b, Tb in enumerate(lens):
        rag.append(0, b, k[b, :Tb], v[b, :Tb], ks, vs)
    assert rag.tokens(0) == lens
    q = np.random.default_rng(4).standard_normal((B, HQ, D)).astype(np.float32)
    for theta in (0.0, 500000.0):
        assert np.array_equal(rag.decode(0, q, rope_theta=theta),
                              full.decode(0, q, rope_theta=theta, seq_tokens=lens))


def test_ragged_kivi_split_follows_each_fill_level():
    """KIVI: a sequence filled to T_b keeps its newest T_b - q(T_b) tokens
    exact in the ring, unlike the prefix of a longer cache (whose rows below
    q(T) are quantised), so the two constructions differ there."""
    T, R = 100, 8
    k, v, ks, vs = _history(acc.KIVI, T, 17)
    lens = [40, 100, 70]
    rag = RaggedCache(acc.KIVI, 2, 1, B, H, D, T, residual=R, in_dtype="f32")
    for b, Tb in enumerate(lens):
        rag.append(0, b, k[b, :Tb], v[b, :Tb])
    kh, vh = rag.seqs[0].dequantized(0)     # 40 tokens: q(40) = 32, 8 exact ring rows
    assert np.array_equal(kh[0, :, 32:40], np.transpose(k[0, 32:40], (1, 0, 2)).astype(np.float64))
    full = OracleCache(acc.KIVI, 2, 1, B, H, D, T, residual=R, in_dtype="f32")
    full.append(0, k, v)
    q = np.random.default_rng(6).standard_normal((B, HQ, D)).astype(np.float32)
    got, pre = rag.decode(0, q), full.decode(0, q, seq_tokens=lens)
    assert np.array_equal(got[1], pre[1])                 # full length: same cache
    assert np.max(np.abs(got[0] - pre[0])) > 1e-4          # 40 of 100: different rows


# ---- several queries per sequence (causal) -----------------------------------

@pytest.mark.parametrize("scheme,bits,R", [(acc.KIVI, 2, 16), (acc.SYM_TOKEN, 4, 0), (acc.BF16_CACHE, 16, 0)])
def test_multi_query_last_is_uniform_decode(scheme, bits, R):
    """The last of n_q queries sees every token: the single-query decode."""
    c, *_, q = filled(scheme, bits, 90, residual=R, seed=21)
    rng = np.random.default_rng(8)
    qm = rng.standard_normal((B, 3, HQ, D)).astype(np.float32)
    qm[:, 2] = q
    for theta in (0.0, 10000.0):
        got = c.decode_multi(0, qm, rope_theta=theta)
        assert np.array_equal(got[:, 2], c.decode(0, q, rope_theta=theta))


def test_multi_query_is_causal_bruteforce():
    """Query i attends to tokens [0, T - n_q + i]: brute force on the
    dequantised rows (a KIVI cache whose queries' tokens sit in the ring)."""
    T, R, nq = 70, 8, 4
    c, *_ = filled(acc.KIVI, 4, T, residual=R, seed=23)
    kh, vh = c.dequantized(0)
    qm = np.random.default_rng(9).standard_normal((B, nq, HQ, D)).astype(np.float32)
    got = c.decode_multi(0, qm)
    sm = 1.0 / np.sqrt(D)
    for b in range(B):
        for i in range(nq):
            n = T - nq + i + 1
            for h in range(HQ):
                g = attention.gqa_kv_head(h, HQ, H)
                want = attention.attend_bruteforce(qm[b, i, h].astype(np.float64), kh[b, g, :n],
                                                   vh[b, g, :n], sm)
                np.testing.assert_allclose(got[b, i, h], want, rtol=0, atol=1e-12)


def test_multi_query_rows_versus_one_query_decodes_at_their_own_fill():
    """Several queries read the KIVI cache as it stands after every token was
    appended. Row i equals a one-query decode of a cache that only ever held
    its first T_i = T - n_q + i + 1 tokens exactly when both fill levels
    quantise the same tokens (q(T_i) == q(T)); where a later flush has encoded
    tokens that the shorter cache still holds in its ring -- or encoded the
    page that holds the query's own token, whose statistics then include later
    tokens -- the rows differ."""
    R, T, nq = 16, 120, 40      # q(T) = 96; fills 81..120 give q = 64 or 96
    c, k, v, _, _, _ = filled(acc.KIVI, 2, T, residual=R, seed=11)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((B, nq, HQ, D)).astype(np.float32)
    got = c.decode_multi(0, q)
    q_all, _ = acc.flush_plan(T, R)
    same = differ = 0
    for i in range(nq):
        Ti = T - nq + i + 1
        short = OracleCache(acc.KIVI, 2, 1, B, H, D, Ti, residual=R, in_dtype="f32")
        short.append(0, k[:, :Ti], v[:, :Ti])
        want = short.decode(0, q[:, i])
        if acc.flush_plan(Ti, R)[0] == q_all:
            assert np.array_equal(got[:, i], want), i
            same += 1
        else:
            assert np.max(np.abs(got[:, i] - want)) > 1e-6, i
            differ += 1
    assert same > 0 and differ > 0
