"""Host logic of bench.py: the algorithmic byte counts its GB/s figures divide
by, checked against the layout sizes the oracle computes independently
(oracle/accounting.py) and against hand counts."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402
from oracle import accounting  # noqa: E402


def test_kivi_page_bytes_match_layout():
    for name in ("kivi2", "int4", "kivi_k4v2", "longctx"):
        w = synth.WORKLOADS[name]
        want = accounting.page_bytes(w.scheme, w.head_dim, w.bits, w.v_bits or None)
        assert bench.kivi_page_bytes(w) == want, name


def test_decode_bytes_hand_count():
    w = synth.WORKLOADS["kivi2"]            # B 16, 8 KV heads, d 128, R 128, 2-bit
    T = 4119                                # q = 3968: 124 pages, 151 ring tokens
    per_unit = 124 * 3328 + 151 * 2 * 128 * 2 + 4 * 128 * (2 + 4)
    assert bench.decode_bytes(w, T) == 16 * 8 * per_unit
    assert bench.decode_bytes(w, T) == 63111168


def test_ragged_decode_bytes():
    w = synth.WORKLOADS["kivi2"]
    T = 4119
    assert bench.ragged_decode_bytes(w, [T] * w.batch) == bench.decode_bytes(w, T)
    qrow = 4 * 128 * (2 + 4)
    # each sequence at its own fill level: 1 token (ring only), 160 tokens
    # (q = 32: one page, 128 ring rows), 4000 tokens (q = 3872: 121 pages,
    # 128 ring rows)
    lens = [1, 160, 4000] + [T] * (w.batch - 3)
    want = 8 * (512 + qrow) + 8 * (3328 + 128 * 512 + qrow) + 8 * (121 * 3328 + 128 * 512 + qrow) \
        + (w.batch - 3) * bench.decode_bytes(w, T) // w.batch
    assert bench.ragged_decode_bytes(w, lens) == want


@pytest.mark.parametrize("T_old,n", [(0, 4096), (4096, 1), (4127, 1), (100, 60)])
def test_append_bytes_flush_accounting(T_old, n):
    """Reads: the new rows plus the ring rows a flush consumes; writes: the
    flushed pages plus the new rows that stay in the ring."""
    w = synth.WORKLOADS["kivi2"]
    R, row, page = w.residual, 2 * 128 * 2, 3328
    q0, q1 = bench.kivi_q(T_old, R), bench.kivi_q(T_old + n, R)
    flushed = q1 - q0
    from_ring = max(0, min(q1, T_old) - q0)
    ring_kept = T_old + n - max(q1, T_old)
    want = (n + from_ring) * row + flushed // 32 * page + ring_kept * row
    assert bench.append_bytes(w, T_old, n) == 16 * 8 * want
    if (T_old, n) == (0, 4096):               # the prefill figure of the bench
        assert bench.append_bytes(w, 0, 4096) == 329646080
