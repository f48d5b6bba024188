"""The C ABI on the host: the library loads, exports what include/kvq.h
declares, sizes agree with the oracle's independent layout arithmetic, and every
validation error is returned before any device work (no GPU needed)."""

import ctypes
import os
import re
import subprocess

import pytest

import kv_cache_quantisation_amd as kvq
from oracle import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"KVQ_API\s+[\w\s\*]+?\b(kvq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = kvq.lib()
    declared = header_functions()
    assert set(declared) == set(kvq.kvq.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.kvq.LIB_PATH],
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)$", out, re.M))
    assert exported == set(declared)     # nothing internal leaks out


def test_abi_version_and_strings():
    assert kvq.kvq_abi_version() == 11
    assert kvq.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5, -6):
        assert kvq.status_string(st) != "unknown status"


def cfg(**kw):
    base = dict(scheme=kvq.KVQ_KIVI, bits=2, layers=2, q_heads=32, kv_heads=8, head_dim=128,
                batch=3, max_tokens=4096, residual=128)
    base.update(kw)
    return kvq.make_config(**base)


def test_struct_layout():
    assert ctypes.sizeof(kvq.kvq_config) == 80
    assert kvq.kvq_config.max_tokens.offset == 32 and kvq.kvq_config.rope_theta.offset == 56
    assert kvq.kvq_config.v_bits.offset == 72
    c = cfg()
    assert kvq.kvq_cache_bytes(c, 10, kvq.KVQ_BYTES_FORMULA) > 0
    c.struct_size = 64
    assert kvq.lib().kvq_cache_bytes(ctypes.byref(c), 10, 0) == kvq.KVQ_ERR_INVALID


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_formula_matches_oracle(bits):
    for scheme in (kvq.KVQ_KIVI, kvq.KVQ_SYM_TOKEN):
        c = cfg(scheme=scheme, bits=bits, residual=128 if scheme == kvq.KVQ_KIVI else 0)
        for T in (0, 1, 4096, 131072):
            assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_FORMULA) == \
                acc.kv_bytes_formula(2, 8, 128, T, bits, batch=3)
    # the page's Llama 3 8B figure through the library: 128 KiB per token at 16 bits
    # is twice the 8-bit formula value
    c = cfg(scheme=kvq.KVQ_FP8_E4M3, bits=8, residual=0, layers=32, batch=1)
    assert 2 * kvq.kvq_cache_bytes(c, 1, kvq.KVQ_BYTES_FORMULA) == 131072
    # and directly for the unquantised bfloat16 cache
    c = cfg(scheme=kvq.KVQ_BF16_CACHE, bits=16, residual=0, layers=32, batch=1)
    assert kvq.kvq_cache_bytes(c, 1, kvq.KVQ_BYTES_FORMULA) == 131072 == \
        acc.kv_bytes_formula(32, 8, 128, 1, 16)


@pytest.mark.parametrize("scheme,bits,d,R,dtype", [
    (kvq.KVQ_KIVI, 2, 128, 128, kvq.KVQ_BF16), (kvq.KVQ_KIVI, 4, 64, 0, kvq.KVQ_F32),
    (kvq.KVQ_KIVI, 8, 256, 37, kvq.KVQ_BF16), (kvq.KVQ_KIVI, 2, 32, 5, kvq.KVQ_F32),
    (kvq.KVQ_SYM_TOKEN, 4, 32, 0, kvq.KVQ_F32), (kvq.KVQ_SYM_TOKEN, 2, 128, 0, kvq.KVQ_BF16),
    (kvq.KVQ_FP8_E4M3, 8, 128, 0, kvq.KVQ_BF16), (kvq.KVQ_BF16_CACHE, 16, 128, 0, kvq.KVQ_BF16),
    (kvq.KVQ_BF16_CACHE, 16, 32, 0, kvq.KVQ_F32), (kvq.KVQ_FP8_E5M2, 8, 64, 0, kvq.KVQ_BF16),
    (kvq.KVQ_KIVI, 3, 128, 128, kvq.KVQ_BF16), (kvq.KVQ_KIVI, 3, 32, 7, kvq.KVQ_F32),
    (kvq.KVQ_SYM_TOKEN, 3, 32, 0, kvq.KVQ_F32), (kvq.KVQ_SYM_TOKEN, 3, 256, 0, kvq.KVQ_BF16)])
def test_cache_bytes_match_oracle_layout(scheme, bits, d, R, dtype):
    c = cfg(scheme=scheme, bits=bits, head_dim=d, residual=R, in_dtype=dtype, q_heads=8)
    item = 2 if dtype == kvq.KVQ_BF16 else 4
    for T in (0, 1, 31, 32, 33, 160, 161, 4096, 10000):
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_CACHE) == \
            acc.layout_cache_bytes(scheme, 2, 3, 8, d, bits, T, R, item), T


@pytest.mark.parametrize("bits,v_bits,d,R,dtype", [
    (4, 2, 128, 128, kvq.KVQ_BF16), (8, 4, 64, 0, kvq.KVQ_F32), (8, 2, 256, 37, kvq.KVQ_BF16),
    (4, 2, 32, 5, kvq.KVQ_F32), (4, 4, 128, 16, kvq.KVQ_BF16), (4, 3, 128, 16, kvq.KVQ_BF16),
    (8, 3, 64, 0, kvq.KVQ_F32), (3, 2, 256, 37, kvq.KVQ_BF16)])
def test_kivi_value_bits_sizes(bits, v_bits, d, R, dtype):
    """KIVI with value codes narrower than key codes: exact layout size and
    the KV-bytes equation with each half at its own width, as the oracle has
    them; v_bits equal to bits is the same cache as v_bits 0."""
    c = cfg(bits=bits, v_bits=v_bits, head_dim=d, residual=R, in_dtype=dtype, q_heads=8)
    item = 2 if dtype == kvq.KVQ_BF16 else 4
    for T in (0, 1, 31, 33, 161, 4096, 10000):
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_CACHE) == \
            acc.layout_cache_bytes(kvq.KVQ_KIVI, 2, 3, 8, d, bits, T, R, item, v_bits), T
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_FORMULA) == \
            acc.kv_bytes_formula(2, 8, d, T, bits, batch=3, v_bits=v_bits)
    if v_bits == bits:
        c0 = cfg(bits=bits, head_dim=d, residual=R, in_dtype=dtype, q_heads=8)
        assert kvq.kvq_cache_bytes(c0, 999, kvq.KVQ_BYTES_CACHE) == \
            kvq.kvq_cache_bytes(c, 999, kvq.KVQ_BYTES_CACHE)


def test_value_bits_validation():
    L = kvq.lib()
    def st(**kw):
        c = cfg(**kw)
        return L.kvq_cache_bytes(ctypes.byref(c), 64, kvq.KVQ_BYTES_CACHE)
    assert st(bits=4, v_bits=2) > 0 and st(bits=8, v_bits=4) > 0 and st(bits=8, v_bits=2) > 0
    assert st(bits=2, v_bits=4) == kvq.KVQ_ERR_UNSUPPORTED     # values wider than keys
    assert st(bits=4, v_bits=8) == kvq.KVQ_ERR_UNSUPPORTED
    assert st(bits=8, v_bits=3) > 0 and st(bits=3, v_bits=2) > 0 and st(bits=3) > 0
    assert st(bits=4, v_bits=3, head_dim=32) == kvq.KVQ_ERR_UNSUPPORTED   # page off 256 bytes
    assert st(bits=3, head_dim=32) > 0
    assert st(scheme=kvq.KVQ_SYM_TOKEN, bits=3, residual=0) > 0
    assert st(bits=3, v_bits=4) == kvq.KVQ_ERR_UNSUPPORTED     # values wider than keys
    assert st(bits=4, v_bits=9) == kvq.KVQ_ERR_INVALID
    assert st(bits=4, v_bits=-2) == kvq.KVQ_ERR_INVALID
    assert st(scheme=kvq.KVQ_SYM_TOKEN, bits=4, v_bits=2, residual=0) == kvq.KVQ_ERR_INVALID
    assert st(scheme=kvq.KVQ_SYM_TOKEN, bits=4, v_bits=4, residual=0) > 0
    assert st(scheme=kvq.KVQ_FP8_E4M3, bits=8, v_bits=4, residual=0) == kvq.KVQ_ERR_INVALID


def test_config_sizes_of_the_workloads():
    # KIVI 2-bit at 4096 tokens: 124 pages of 104 B/token-head + a 160-row bf16 ring
    c = cfg(batch=16, layers=1)
    assert kvq.kvq_cache_bytes(c, 4096, kvq.KVQ_BYTES_CACHE) == 16 * 8 * (124 * 3328 + 81920)


def test_workspace_monotone():
    c = cfg()
    prev = 0
    for T in list(range(1, 400)) + [4096, 100000, 1 << 20]:
        w = kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_WORKSPACE)
        assert w >= prev
        prev = w
    c.num_splits = 3
    assert kvq.kvq_cache_bytes(c, 4096, kvq.KVQ_BYTES_WORKSPACE) >= 3 * 32 * 3 * 130 * 4


@pytest.mark.parametrize("field,value,status", [
    ("scheme", 7, kvq.KVQ_ERR_INVALID), ("bits", 5, kvq.KVQ_ERR_UNSUPPORTED),
    ("bits", 0, kvq.KVQ_ERR_INVALID), ("bits", 16, kvq.KVQ_ERR_INVALID),
    ("layers", 0, kvq.KVQ_ERR_INVALID), ("q_heads", 12, kvq.KVQ_ERR_INVALID),
    ("q_heads", 8 * 16, kvq.KVQ_ERR_UNSUPPORTED), ("q_heads", 8 * 3, kvq.KVQ_ERR_UNSUPPORTED),
    ("head_dim", 96, kvq.KVQ_ERR_UNSUPPORTED), ("head_dim", 0, kvq.KVQ_ERR_INVALID),
    ("group", 64, kvq.KVQ_ERR_UNSUPPORTED), ("group", 0, kvq.KVQ_ERR_INVALID),
    ("residual", -1, kvq.KVQ_ERR_INVALID), ("in_dtype", 5, kvq.KVQ_ERR_INVALID),
    ("q_dtype", -1, kvq.KVQ_ERR_INVALID), ("rope_theta", -1.0, kvq.KVQ_ERR_INVALID),
    ("rope_theta", float("nan"), kvq.KVQ_ERR_INVALID), ("sm_scale", float("inf"), kvq.KVQ_ERR_INVALID),
    ("num_splits", -2, kvq.KVQ_ERR_INVALID), ("batch", 0, kvq.KVQ_ERR_INVALID),
    ("batch", 70000, kvq.KVQ_ERR_UNSUPPORTED), ("max_tokens", -5, kvq.KVQ_ERR_INVALID),
    ("max_tokens", 1 << 40, kvq.KVQ_ERR_UNSUPPORTED)])
def test_config_validation(field, value, status):
    c = cfg()
    setattr(c, field, value)
    L = kvq.lib()
    assert L.kvq_cache_bytes(ctypes.byref(c), 8, 1) == status
    # the same status comes back from both device entry points, before any launch
    fake = 1 << 20
    assert L.kvq_quantize_append(ctypes.byref(c), fake, 0, 0, 4, fake, fake, None, None, None) \
        == status
    assert L.kvq_decode_attention(ctypes.byref(c), fake, 0, 8, fake, None, None, fake, fake,
                                  1 << 30, None) == status


def test_scheme_specific_validation():
    L = kvq.lib()
    c = cfg(scheme=kvq.KVQ_SYM_TOKEN, bits=4, residual=3)
    assert L.kvq_cache_bytes(ctypes.byref(c), 8, 1) == kvq.KVQ_ERR_INVALID
    c = cfg(scheme=kvq.KVQ_FP8_E4M3, bits=4, residual=0)
    assert L.kvq_cache_bytes(ctypes.byref(c), 8, 1) == kvq.KVQ_ERR_INVALID
    for bits, R in ((8, 0), (2, 0), (16, 4)):      # bfloat16 cache: bits 16, no residual
        c = cfg(scheme=kvq.KVQ_BF16_CACHE, bits=bits, residual=R)
        assert L.kvq_cache_bytes(ctypes.byref(c), 8, 1) == kvq.KVQ_ERR_INVALID
    c = cfg(scheme=kvq.KVQ_BF16_CACHE, bits=16, residual=0)
    assert L.kvq_cache_bytes(ctypes.byref(c), 64, 1) == 2 * 3 * 8 * 2 * 128 * 32 * 4
    for bits in (4, 16):                                 # E5M2: bits 8
        c = cfg(scheme=kvq.KVQ_FP8_E5M2, bits=bits, residual=0)
        assert L.kvq_cache_bytes(ctypes.byref(c), 8, 1) == kvq.KVQ_ERR_INVALID
    c = cfg(scheme=kvq.KVQ_FP8_E5M2, bits=8, residual=0)
    fake = 1 << 20                                       # and needs its scales
    assert L.kvq_quantize_append(ctypes.byref(c), fake, 0, 0, 4, fake, fake, None, fake, None) \
        == kvq.KVQ_ERR_NULL
    assert L.kvq_decode_attention(ctypes.byref(c), fake, 0, 8, fake, None, fake, fake, fake,
                                  1 << 30, None) == kvq.KVQ_ERR_NULL
    c = cfg(scheme=kvq.KVQ_FP8_E4M3, bits=8, residual=0)
    fake = 1 << 20
    # FP8 needs its per-head scales
    assert L.kvq_quantize_append(ctypes.byref(c), fake, 0, 0, 4, fake, fake, None, None, None) \
        == kvq.KVQ_ERR_NULL
    assert L.kvq_decode_attention(ctypes.byref(c), fake, 0, 8, fake, fake, None, fake, fake,
                                  1 << 30, None) == kvq.KVQ_ERR_NULL
    assert L.kvq_cache_bytes(ctypes.byref(c), 8, 9) == kvq.KVQ_ERR_INVALID
    assert L.kvq_cache_bytes(ctypes.byref(c), -1, 1) == kvq.KVQ_ERR_INVALID
    assert L.kvq_cache_bytes(None, 8, 1) == kvq.KVQ_ERR_NULL


def test_call_validation():
    L = kvq.lib()
    c = cfg()
    p = ctypes.byref(c)
    f = 1 << 20
    big = 1 << 30
    ap = L.kvq_quantize_append
    assert ap(None, f, 0, 0, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ap(p, None, 0, 0, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ap(p, f, 2, 0, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID      # layer
    assert ap(p, f, -1, 0, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID
    assert ap(p, f, 0, -1, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID
    assert ap(p, f, 0, 4000, 97, f, f, None, None, None) == kvq.KVQ_ERR_CAPACITY
    assert ap(p, f, 0, 4097, 0, f, f, None, None, None) == kvq.KVQ_ERR_CAPACITY
    assert ap(p, f, 0, 4000, 0, None, None, None, None, None) == kvq.KVQ_OK       # no-op
    assert ap(p, f, 0, 0, 4, None, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ap(p, f + 4, 0, 0, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID  # alignment
    assert ap(p, f, 0, 0, 4, f + 2, f, None, None, None) == kvq.KVQ_ERR_INVALID
    de = L.kvq_decode_attention
    assert de(p, f, 0, 0, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID   # tokens
    assert de(p, f, 0, 4097, f, None, None, f, f, big, None) == kvq.KVQ_ERR_CAPACITY
    assert de(p, f, 0, 8, None, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert de(p, f, 0, 8, f, None, None, None, f, big, None) == kvq.KVQ_ERR_NULL
    assert de(p, f, 0, 8, f, None, None, f, None, big, None) == kvq.KVQ_ERR_NULL
    assert de(p, f, 0, 8, f, None, None, f + 8, f, big, None) == kvq.KVQ_ERR_INVALID
    need = kvq.kvq_cache_bytes(c, 4096, kvq.KVQ_BYTES_WORKSPACE)
    assert de(p, f, 0, 4096, f, None, None, f, f, need - 1, None) == kvq.KVQ_ERR_WORKSPACE
    assert de(p, f, 3, 8, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID    # layer


def test_ragged_call_validation():
    """The ragged decode validates as kvq_decode_attention does, and needs its
    per-sequence counts (a device array: present and 8-byte aligned)."""
    L = kvq.lib()
    c = cfg()
    p = ctypes.byref(c)
    f = 1 << 20
    big = 1 << 30
    rd = L.kvq_decode_attention_ragged
    assert rd(p, f, 0, 8, None, f, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert rd(p, f, 0, 8, f + 4, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert rd(None, f, 0, 8, f, f, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert rd(p, f, 0, 0, f, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert rd(p, f, 0, 4097, f, f, None, None, f, f, big, None) == kvq.KVQ_ERR_CAPACITY
    assert rd(p, f, 0, 8, f, None, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert rd(p, f, 3, 8, f, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    need = kvq.kvq_cache_bytes(c, 4096, kvq.KVQ_BYTES_WORKSPACE)
    assert rd(p, f, 0, 4096, f, f, None, None, f, f, need - 1, None) == kvq.KVQ_ERR_WORKSPACE


def test_ragged_append_validation():
    """The ragged append validates as kvq_quantize_append does, and needs its
    per-sequence counts (device arrays: present and 8-byte aligned)."""
    L = kvq.lib()
    c = cfg()
    p = ctypes.byref(c)
    f = 1 << 20
    ra = L.kvq_quantize_append_ragged
    assert ra(None, f, 0, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ra(p, None, 0, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ra(p, f, 0, None, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ra(p, f, 0, f, None, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ra(p, f, 0, f, f, 4, None, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ra(p, f, 2, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID     # layer
    assert ra(p, f, 0, f, f, -1, f, f, None, None, None) == kvq.KVQ_ERR_INVALID    # bound
    assert ra(p, f, 0, f, f, 4097, f, f, None, None, None) == kvq.KVQ_ERR_CAPACITY
    assert ra(p, f, 0, f + 4, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID  # alignment
    assert ra(p, f, 0, f, f, 4, f + 2, f, None, None, None) == kvq.KVQ_ERR_INVALID
    assert ra(p, f, 0, None, None, 0, None, None, None, None, None) == kvq.KVQ_OK   # no-op


def test_multi_query_validation():
    """Several queries per sequence: 1 <= n_queries <= tokens, and a workspace
    of n_queries single-query workspaces."""
    L = kvq.lib()
    c = cfg()
    p = ctypes.byref(c)
    f = 1 << 20
    big = 1 << 30
    mq = L.kvq_decode_attention_multi
    assert mq(p, f, 0, 8, 0, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert mq(p, f, 0, 8, 9, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert mq(p, f, 0, 8, 2, None, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert mq(p, f, 0, 0, 1, f, None, None, f, f, big, None) == kvq.KVQ_ERR_INVALID
    need = kvq.kvq_cache_bytes(c, 4096, kvq.KVQ_BYTES_WORKSPACE)
    assert mq(p, f, 0, 4096, 3, f, None, None, f, f, 3 * need - 1, None) == kvq.KVQ_ERR_WORKSPACE
    # one row of blocks per (sequence, query): batch * n_queries <= 65535,
    # checked in 64-bit before any launch
    # (a zero workspace stops the allowed case at the next check, before any launch)
    c.batch = 4096
    c.max_tokens = 64
    assert mq(p, f, 0, 64, 15, f, None, None, f, f, 0, None) == kvq.KVQ_ERR_WORKSPACE
    assert mq(p, f, 0, 64, 16, f, None, None, f, f, 0, None) == kvq.KVQ_ERR_UNSUPPORTED


def test_noalloc_validation():
    """The decode without a workspace validates on the host before touching a
    device: bad arguments, and a call whose workspace need exceeds the
    library's scratch array (KVQ_ERR_WORKSPACE)."""
    L = kvq.lib()
    f = 1 << 20
    c = cfg()
    p = ctypes.byref(c)
    na = L.kvq_decode_attention_noalloc
    assert na(None, f, 0, 8, f, None, None, f, None) == kvq.KVQ_ERR_NULL
    assert na(p, None, 0, 8, f, None, None, f, None) == kvq.KVQ_ERR_NULL
    assert na(p, f, 0, 8, f, None, None, None, None) == kvq.KVQ_ERR_NULL
    assert na(p, f, 2, 8, f, None, None, f, None) == kvq.KVQ_ERR_INVALID       # layer
    assert na(p, f, 0, 0, f, None, None, f, None) == kvq.KVQ_ERR_INVALID       # tokens
    assert na(p, f, 0, 4097, f, None, None, f, None) == kvq.KVQ_ERR_CAPACITY
    assert na(p, f + 8, 0, 8, f, None, None, f, None) == kvq.KVQ_ERR_INVALID   # alignment
    # a workspace need beyond the scratch array: many sequences, many splits
    big = cfg(batch=4096, max_tokens=1 << 16, num_splits=64)
    need = kvq.kvq_cache_bytes(big, 1 << 16, kvq.KVQ_BYTES_WORKSPACE)
    assert need > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert na(ctypes.byref(big), f, 0, 1 << 16, f, None, None, f, None) == kvq.KVQ_ERR_WORKSPACE


@pytest.mark.parametrize("bits,v_bits,d,R,dtype", [
    (2, 0, 128, 128, kvq.KVQ_BF16), (4, 2, 64, 0, kvq.KVQ_F32), (8, 0, 256, 37, kvq.KVQ_BF16),
    (2, 0, 32, 5, kvq.KVQ_F32)])
def test_sparse_outlier_sizes_and_validation(bits, v_bits, d, R, dtype):
    """Dense-and-sparse KIVI pages: each page grows by its side matrix
    (5 d + 160 bytes, padded to 256) exactly as the oracle's layout has it;
    only KIVI takes outliers, and only 0 or 1."""
    c = cfg(bits=bits, v_bits=v_bits, head_dim=d, residual=R, in_dtype=dtype, q_heads=8,
            outliers=1)
    item = 2 if dtype == kvq.KVQ_BF16 else 4
    for T in (0, 1, 31, 33, 161, 4096, 10000):
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_CACHE) == \
            acc.layout_cache_bytes(kvq.KVQ_KIVI, 2, 3, 8, d, bits, T, R, item, v_bits or None,
                                   outliers=1), T
    L = kvq.lib()
    def st(**kw):
        return L.kvq_cache_bytes(ctypes.byref(cfg(**kw)), 64, kvq.KVQ_BYTES_CACHE)
    assert st(outliers=2) == kvq.KVQ_ERR_INVALID
    assert st(outliers=-1) == kvq.KVQ_ERR_INVALID
    assert st(scheme=kvq.KVQ_SYM_TOKEN, bits=4, residual=0, outliers=1) == kvq.KVQ_ERR_INVALID
    assert st(scheme=kvq.KVQ_FP8_E4M3, bits=8, residual=0, outliers=1) == kvq.KVQ_ERR_INVALID


def test_paged_sizes_and_validation():
    """Paged caches: size = ring region (256-aligned) + blocks, as the oracle's
    paged image has it; the table is checked on the host (null, alignment,
    a row too short for a full sequence, block counts) before any launch."""
    from oracle.cache import OracleCache, paged_image
    import numpy as np
    L = kvq.lib()
    c = cfg(batch=2, max_tokens=200, residual=16, head_dim=32, q_heads=8, in_dtype=kvq.KVQ_F32)
    oc = OracleCache(kvq.KVQ_KIVI, 2, 2, 2, 8, 32, 200, residual=16, in_dtype="f32")
    P = (200 - 16) // 32
    for nb in (2 * P, 2 * P + 5):
        buf, _ = paged_image(oc, np.arange(2 * P).reshape(2, P), nb)
        assert kvq.kvq_paged_cache_bytes(c, nb) == buf.size
    p = ctypes.byref(c)
    f = 1 << 20
    ap = L.kvq_quantize_append_paged
    dp = L.kvq_decode_attention_paged
    assert ap(p, f, 0, None, P, 10, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_NULL
    assert ap(p, f, 0, f + 2, P, 10, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID
    assert ap(p, f, 0, f, P - 1, 10, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_CAPACITY
    assert ap(p, f, 0, f, P, 0, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_INVALID
    assert ap(p, f, 0, f, P, 1 << 31, f, f, 4, f, f, None, None, None) == kvq.KVQ_ERR_UNSUPPORTED
    assert ap(p, f, 0, f, P, 10, f, f, 0, f, f, None, None, None) == kvq.KVQ_OK    # no-op
    assert dp(p, f, 0, None, P, 10, 8, f, f, None, None, f, f, 1 << 20, None) == kvq.KVQ_ERR_NULL
    assert dp(p, f, 0, f, P - 1, 10, 8, f, f, None, None, f, f, 1 << 20, None) == kvq.KVQ_ERR_CAPACITY
    assert dp(p, f, 0, f, P, 10, 8, None, f, None, None, f, f, 1 << 20, None) == kvq.KVQ_ERR_NULL
    assert dp(p, f, 0, f, P, 10, 8, f, f, None, None, f, f, 0, None) == kvq.KVQ_ERR_WORKSPACE
    assert L.kvq_paged_cache_bytes(p, -1) == kvq.KVQ_ERR_INVALID


def test_append_decode_validation():
    """kvq_append_decode checks both calls' arguments before launching."""
    L = kvq.lib()
    c = cfg()
    p = ctypes.byref(c)
    f = 1 << 20
    big = 1 << 30
    ad = L.kvq_append_decode
    assert ad(None, f, 0, 8, f, f, None, None, f, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert ad(p, f, 0, -1, f, f, None, None, f, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert ad(p, f, 0, 4096, f, f, None, None, f, f, f, big, None) == kvq.KVQ_ERR_CAPACITY
    assert ad(p, f, 0, 8, None, f, None, None, f, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert ad(p, f, 0, 8, f, f + 4, None, None, f, f, f, big, None) == kvq.KVQ_ERR_INVALID
    assert ad(p, f, 0, 8, f, f, None, None, None, f, f, big, None) == kvq.KVQ_ERR_NULL
    assert ad(p, f, 0, 8, f, f, None, None, f, f, f, 0, None) == kvq.KVQ_ERR_WORKSPACE
    assert ad(p, f, 5, 8, f, f, None, None, f, f, f, big, None) == kvq.KVQ_ERR_INVALID   # layer


@pytest.mark.parametrize("vb,d,dtype", [(2, 128, kvq.KVQ_BF16), (3, 64, kvq.KVQ_F32), (4, 32, kvq.KVQ_BF16),
                                        (8, 256, kvq.KVQ_F32), (0, 64, kvq.KVQ_BF16)])
@pytest.mark.parametrize("scheme", ["symv", "kiviv"])
def test_fp8k_mixed_sizes(vb, d, dtype, scheme):
    """FP8 keys with symmetric or KIVI values: layout size and KV-bytes equation (keys
    at 8 bits, values at v_bits; v_bits 0 means 8) as the oracle has them;
    every page a multiple of 256 bytes."""
    sch = {"symv": (kvq.KVQ_FP8K_SYMV, acc.FP8K_SYMV), "kiviv": (kvq.KVQ_FP8K_KIVIV, acc.FP8K_KIVIV)}[scheme]
    c = cfg(scheme=sch[0], bits=8, v_bits=vb, head_dim=d, residual=0, in_dtype=dtype,
            q_heads=8)
    v = vb or 8
    item = 2 if dtype == kvq.KVQ_BF16 else 4
    assert acc.page_bytes(sch[1], d, 8, v) % 256 == 0
    for T in (0, 1, 31, 32, 33, 161, 4096):
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_CACHE) == \
            acc.layout_cache_bytes(sch[1], 2, 3, 8, d, 8, T, 0, item, v), T
        assert kvq.kvq_cache_bytes(c, T, kvq.KVQ_BYTES_FORMULA) == \
            acc.kv_bytes_formula(2, 8, d, T, 8, batch=3, v_bits=v)


@pytest.mark.parametrize("scheme", ["symv", "kiviv"])
def test_fp8k_mixed_validation(scheme):
    L = kvq.lib()
    def st(**kw):
        base = dict(scheme=kvq.KVQ_FP8K_SYMV if scheme == "symv" else kvq.KVQ_FP8K_KIVIV, bits=8, residual=0)
        base.update(kw)
        c = cfg(**base)
        return L.kvq_cache_bytes(ctypes.byref(c), 64, kvq.KVQ_BYTES_CACHE)
    assert all(st(v_bits=v) > 0 for v in (0, 2, 3, 4, 8))
    assert st(bits=4) == kvq.KVQ_ERR_INVALID                  # keys are FP8: 8 bits
    assert st(v_bits=5) == kvq.KVQ_ERR_UNSUPPORTED and st(v_bits=9) == kvq.KVQ_ERR_INVALID
    assert st(v_bits=3, head_dim=32) == kvq.KVQ_ERR_UNSUPPORTED
    assert st(residual=16) == kvq.KVQ_ERR_INVALID              # no residual ring
    assert st(outliers=1) == kvq.KVQ_ERR_INVALID


@pytest.mark.parametrize("scheme", ["symv", "kiviv"])
def test_fp8k_mixed_needs_the_key_scale_only(scheme):
    """The key scale is required (KVQ_ERR_NULL without it, nothing launched);
    the value scale is not read (validation passes it as NULL and stops at the
    next check, a null cache)."""
    L = kvq.lib()
    c = cfg(scheme=kvq.KVQ_FP8K_SYMV if scheme == "symv" else kvq.KVQ_FP8K_KIVIV, bits=8, v_bits=4,
            residual=0)
    fake = ctypes.c_void_p(16)
    ks = ctypes.cast(ctypes.c_void_p(16), ctypes.POINTER(ctypes.c_float))
    nul = ctypes.POINTER(ctypes.c_float)()
    odd = ctypes.c_void_p(8)                                   # fails the alignment check
    st = L.kvq_quantize_append(ctypes.byref(c), fake, 0, 0, 4, odd, fake, nul, nul, None)
    assert st == kvq.KVQ_ERR_NULL
    st = L.kvq_quantize_append(ctypes.byref(c), fake, 0, 0, 4, odd, fake, ks, nul, None)
    assert st == kvq.KVQ_ERR_INVALID                           # past the scale checks
    out = ctypes.cast(fake, ctypes.POINTER(ctypes.c_float))
    st = L.kvq_decode_attention(ctypes.byref(c), fake, 0, 64, fake, nul, nul, out, fake, 0, None)
    assert st == kvq.KVQ_ERR_NULL
    st = L.kvq_decode_attention(ctypes.byref(c), fake, 0, 64, fake, ks, nul, out, fake, 0, None)
    assert st == kvq.KVQ_ERR_WORKSPACE                         # past the scale checks
