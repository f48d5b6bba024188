"""Pins of oracle.accounting against numbers the pages print."""

import pytest

from oracle import accounting as acc

GIB = 2 ** 30


def test_llama3_bytes_per_token(golden):
    g = golden("pages_memory.json")["llama3_8b"]
    sh = g["shape"]
    assert acc.kv_bytes_formula(sh["layers"], sh["kv_heads"], sh["head_dim"], 1, 16) == \
        g["bytes_per_token_16bit"]
    assert acc.kv_bytes_formula(sh["layers"], sh["kv_heads"], sh["head_dim"], 128 * 1024, 16) == \
        g["tokens_128k_16bit_gib"] * GIB
    # FP8 halves, 4 bits quarters
    b16 = acc.kv_bytes_formula(32, 8, 128, 1000, 16)
    assert acc.kv_bytes_formula(32, 8, 128, 1000, 8) * 2 == b16
    assert acc.kv_bytes_formula(32, 8, 128, 1000, 4) * 4 == b16


def test_long_context_example(golden):
    g = golden("pages_memory.json")["long_context_example"]
    for bits, gib in g["gib"].items():
        assert acc.kv_bytes_formula(32, 8, 128, g["context"], int(bits), batch=g["users"]) == gib * GIB


def test_widget(golden):
    g = golden("pages_memory.json")["widget"]
    total = acc.kv_bytes_formula(32, 8, 128, g["context"], 16, batch=g["users"])
    assert total / GIB == pytest.approx(g["kv_gib"], abs=0.05)
    assert acc.kv_bytes_formula(32, 8, 128, 1, 16) == g["kv_per_token_kib"] * 1024


def test_llama7b_glossary(golden):
    g = golden("pages_memory.json")["llama7b_glossary"]
    sh = g["shape"]
    per_tok = acc.kv_bytes_formula(sh["layers"], sh["kv_heads"], sh["head_dim"], 1, 16)
    assert per_tok == g["bytes_per_token_fp16"]
    assert acc.kv_bytes_formula(32, 32, 128, 2048, 16) == g["tokens_2048_gib"] * GIB
    assert acc.kv_bytes_formula(32, 32, 128, 2048, 16, batch=32) == g["batch32_tokens_2048_gib"] * GIB


def test_gqa_ratio(golden):
    g = golden("pages_memory.json")["gqa"]
    with_gqa = acc.kv_bytes_formula(32, 8, 128, 4096, 16)
    without = acc.kv_bytes_formula(32, 32, 128, 4096, 16)
    assert without == g["ratio_without_gqa"] * with_gqa


def test_formula_scales_linearly():
    # The cache grows linearly with context and with conversations served.
    a = acc.kv_bytes_formula(4, 2, 64, 100, 8)
    assert acc.kv_bytes_formula(4, 2, 64, 300, 8) == 3 * a
    assert acc.kv_bytes_formula(4, 2, 64, 100, 8, batch=5) == 5 * a
    assert acc.kv_bytes_formula(4, 2, 64, 100, 2) * 4 == a


def test_concurrency(golden):
    g = golden("pages_memory.json")["concurrency"]
    for bits, n in g["conversations"].items():
        assert acc.concurrency(int(bits), gpu_bytes=g["gpu_bytes"], use=g["use"],
                               weight_bytes=g["weight_bytes"], context=g["context"]) == n


def test_concurrency_reading_is_unique():
    # Other readings of "80 GB at 90% use" give numbers the page does not print.
    per_tok = acc.kv_bytes_formula(32, 8, 128, 1, 16) * 8192
    assert int(((80e9 - 16.1e9) * 0.9) // per_tok) == 53
    assert int((0.9 * 80 * GIB - 16.1 * GIB) // per_tok) == 55


def test_flush_plan_closed_form():
    R, G = 128, 32
    for T in range(0, 600):
        q, n_r = acc.flush_plan(T, R, G)
        assert q % G == 0 and q + n_r == T
        if T < R:
            assert (q, n_r) == (0, T)
        else:
            assert n_r == R + (T - R) % G
            assert R <= n_r < R + G
    # the KIVI configs: 4096 and 32768 tokens keep exactly 128 in the window
    assert acc.flush_plan(4096, 128) == (3968, 128)
    assert acc.flush_plan(32768, 128) == (32640, 128)
    assert acc.flush_plan(1048576, 128) == (1048448, 128)
    assert acc.flush_plan(100, 0) == (96, 4)


def test_scale_overhead_half_bit(golden):
    g = golden("pages_memory.json")["scale_overhead_per_token_value"]
    # values per token: one fp32 scale + one fp32 offset per 128-value row
    d = 128
    kivi2 = acc.page_bytes(acc.KIVI, d, 2)
    v_meta_bits = 8 * (4 * 32 + 4 * 32)
    assert v_meta_bits / (32 * d) == g["bits_per_value"]
    # page = codes at 2 bits for K and V + metadata
    assert kivi2 == 2 * 32 * d * 2 // 8 + 8 * d + 256


def test_layout_sizes():
    # KIVI at d=128: 104 / 168 / 296 bytes per token, FP8 256, SYM 4-bit d=32 40
    assert acc.page_bytes(acc.KIVI, 128, 2) == 104 * 32
    assert acc.page_bytes(acc.KIVI, 128, 4) == 168 * 32
    assert acc.page_bytes(acc.KIVI, 128, 8) == 296 * 32
    assert acc.page_bytes(acc.FP8_E4M3, 128, 8) == 256 * 32
    assert acc.page_bytes(acc.SYM_TOKEN, 32, 4) == 40 * 32
    assert acc.page_bytes(acc.BF16_CACHE, 128, 16) == 512 * 32      # 2 x 128 x 2 bytes per token
    assert acc.page_bytes(acc.FP8_E5M2, 128, 8) == acc.page_bytes(acc.FP8_E4M3, 128, 8)
    for s in (acc.KIVI, acc.SYM_TOKEN):
        for d in (32, 64, 128, 256):
            for b in (2, 4, 8):
                assert acc.page_bytes(s, d, b) % 256 == 0
    # capacity 4096 tokens, R=128: 124 pages + ring of 160 bf16 rows for K and V
    assert acc.slab_bytes(acc.KIVI, 128, 2, 4096, 128, 2) == 124 * 3328 + 2 * 160 * 128 * 2
    assert acc.pages_per_slab(acc.SYM_TOKEN, 513, 0) == 17
    assert acc.layout_cache_bytes(acc.FP8_E4M3, 2, 3, 4, 128, 8, 64, 0, 2) == 2 * 3 * 4 * 2 * 8192


def test_value_bits_accounting(golden):
    """Keys and values at their own widths ("Quantizing the KV cache", How the
    KV cache is quantized: separate key and value cache types): each half of
    the KV-bytes equation at its own width. Llama 3 8B's 128 KiB per token at
    16 bits gives 24 KiB with 4-bit keys and 2-bit values (6/32 of it), half
    way between the 4-bit and the 2-bit cache."""
    g = golden("pages_memory.json")["llama3_8b"]
    sh = g["shape"]
    per16 = g["bytes_per_token_16bit"]
    mixed = acc.kv_bytes_formula(sh["layers"], sh["kv_heads"], sh["head_dim"], 1, 4, v_bits=2)
    assert mixed * 32 == per16 * 6 == 24 * 1024 * 32
    assert 2 * mixed == acc.kv_bytes_formula(32, 8, 128, 1, 4) + acc.kv_bytes_formula(32, 8, 128, 1, 2)
    assert acc.kv_bytes_formula(32, 8, 128, 77, 8, v_bits=8) == acc.kv_bytes_formula(32, 8, 128, 77, 8)
    # a KIVI page with 4-bit keys and 2-bit values: 2048 B of key codes, 1024 B
    # of value codes, 1024 B of key scale/offset, 256 B of value scale/offset
    assert acc.page_bytes(acc.KIVI, 128, 4, 2) == 2048 + 1024 + 1024 + 256
    for d in (32, 64, 128, 256):
        for kb, vb in ((4, 2), (8, 2), (8, 4)):
            p = acc.page_bytes(acc.KIVI, d, kb, vb)
            assert p % 256 == 0
            assert 2 * p == acc.page_bytes(acc.KIVI, d, kb) + acc.page_bytes(acc.KIVI, d, vb)
