"""Pins of oracle.attention and oracle.rope: brute force, closed forms, invariants."""

import math

import numpy as np
import pytest

from oracle import attention, rope


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("T,d", [(1, 2), (5, 4), (17, 8), (64, 8)])
def test_attend_matches_bruteforce(T, d):
    q, k, v = _rand(T, d), _rand(T + 1, T, d), _rand(T + 2, T, d)
    sm = 1 / math.sqrt(d)
    assert np.allclose(attention.attend(q, k, v, sm), attention.attend_bruteforce(q, k, v, sm),
                       rtol=0, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((9, 6))
    q = rng.standard_normal(6)
    same_k = np.tile(rng.standard_normal(6), (9, 1))
    assert np.allclose(attention.attend(q, same_k, v, 0.3), v.mean(axis=0), atol=1e-14)
    assert np.allclose(attention.attend(np.zeros(6), rng.standard_normal((9, 6)), v, 0.3),
                       v.mean(axis=0), atol=1e-14)
    assert np.allclose(attention.attend(q, rng.standard_normal((1, 6)), v[:1], 0.3), v[0],
                       atol=1e-15)
    # one key far more aligned than the rest: output -> that value row
    k = rng.standard_normal((9, 6)) * 0.01
    k[4] = q * 100
    assert np.allclose(attention.attend(q, k, v, 1.0), v[4], atol=1e-12)


def test_attend_scale_matters():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal(4), rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    a = attention.attend(q, k, v, 0.5)
    b = attention.attend(q * 0.5, k, v, 1.0)
    assert np.allclose(a, b, atol=1e-14)
    assert not np.allclose(a, attention.attend(q, k, v, 1.0), atol=1e-3)


@pytest.mark.parametrize("bounds", [[0, 40], [0, 1, 40], [0, 13, 14, 27, 40], [0, 32, 40]])
def test_split_merge_equals_one_pass(bounds):
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal(8) * 3, rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    assert np.allclose(attention.split_merge(q, k, v, 0.35, bounds),
                       attention.attend(q, k, v, 0.35), atol=1e-12)


def test_gqa_mapping():
    # 32 query heads over 8 KV heads: heads 0-3 -> 0, 4-7 -> 1, ..., 28-31 -> 7
    assert [attention.gqa_kv_head(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [attention.gqa_kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 4, 8))
    k = rng.standard_normal((2, 2, 10, 8))
    v = rng.standard_normal((2, 2, 10, 8))
    out = attention.decode(q, k, v, 0.3)
    assert np.allclose(out[1, 3], attention.attend(q[1, 3], k[1, 1], v[1, 1], 0.3))
    assert np.allclose(out[0, 1], attention.attend(q[0, 1], k[0, 0], v[0, 0], 0.3))


# ---- rotary embedding ------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = _rand(5, 3, 16)
    assert np.array_equal(rope.rotate(x, np.zeros(3), 500000.0), x)


def test_rope_d2_closed_form():
    # d = 2: a single pair with frequency theta^0 = 1, angle = position
    x = np.array([[1.0, 0.0], [0.3, -2.0]])
    pos = np.array([math.pi / 2, 1.25])
    out = rope.rotate(x, pos, 10000.0)
    assert np.allclose(out[0], [0.0, 1.0], atol=1e-15)
    c, s = math.cos(1.25), math.sin(1.25)
    assert np.allclose(out[1], [0.3 * c + 2.0 * s, 0.3 * s - 2.0 * c], atol=1e-15)


def test_rope_frequencies():
    w = rope.frequencies(8, 10000.0)
    assert np.allclose(w, [1.0, 10000 ** -0.25, 10000 ** -0.5, 10000 ** -0.75])


def test_rope_preserves_norm_and_pairs():
    x = _rand(6, 7, 128)
    pos = np.arange(7) * 1234567.0
    y = rope.rotate(x, pos, 500000.0)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    pair_norm = lambda a: a[:, 0::2] ** 2 + a[:, 1::2] ** 2   # noqa: E731
    assert np.allclose(pair_norm(y), pair_norm(x), rtol=1e-12)


def test_rope_scores_depend_on_relative_position():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal(64), rng.standard_normal((5, 64))
    t = np.array([0, 3, 100, 9999, 123456])
    T = 200000

    def scores(shift):
        kr = rope.rotate(k, t + shift, 500000.0)
        qr = rope.rotate(q, np.float64(T - 1 + shift), 500000.0)
        return kr @ qr
    assert np.allclose(scores(0), scores(777), atol=1e-9)
    assert np.allclose(scores(0), scores(1 << 19), atol=1e-9)
    # and the rotation is not a no-op
    assert not np.allclose(scores(0), k @ q, atol=1e-3)
