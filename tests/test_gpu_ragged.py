"""GPU parity of the ragged-batch decode (kvq_decode_attention_ragged): every
sequence attends to its own first T_b cached tokens, compared with the oracle's
ragged decode (float64) on the same seeded inputs. The lengths put sequences
on one token, inside a page, on a page boundary, inside the KIVI ring and at
the fill level, on every decode kernel (8- and 4-wave KIVI matrix-core, rotary
GQA-4, FP8 / bfloat16 pages, the generic kernel)."""

import numpy as np
import pytest
import torch

import kv_cache_quantisation_amd as kvq
import synth
import harness as H
from test_gpu_parity import run_append, small

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)

CASES = [
    # scheme, bits, d, hg, dtype, R, T, rope, splits
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 700, 0.0, 0),      # 8-wave matrix-core
    (synth.KIVI, 2, 64, 2, torch.float32, 0, 257, 0.0, 5),
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 128, 700, 0.0, 3),      # 4-wave matrix-core
    (synth.KIVI, 2, 128, 8, torch.bfloat16, 40, 450, 0.0, 0),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 700, 500000.0, 0),  # rotary, GQA 4
    (synth.KIVI, 2, 128, 2, torch.bfloat16, 40, 1000, 500000.0, 5),  # rotary, other GQA
    (synth.KIVI, 8, 128, 8, torch.bfloat16, 16, 333, 0.0, 0),       # generic
    (synth.KIVI, 4, 32, 1, torch.float32, 3, 98, 0.0, 0),
    (synth.KIVI, 4, 64, 2, torch.bfloat16, 20, 250, 10000.0, 4),
    (synth.SYM_TOKEN, 4, 32, 1, torch.float32, 0, 512, 0.0, 0),
    (synth.SYM_TOKEN, 4, 256, 2, torch.bfloat16, 0, 200, 500000.0, 3),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 333, 0.0, 0),    # FP8 pages
    (synth.FP8_E5M2, 8, 64, 2, torch.bfloat16, 0, 97, 0.0, 3),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 300, 500000.0, 0),
    (synth.BF16_CACHE, 16, 128, 4, torch.bfloat16, 0, 333, 0.0, 0),  # bfloat16 pages
    (synth.BF16_CACHE, 16, 256, 2, torch.bfloat16, 0, 200, 500000.0, 3),
]


def lengths(T, R, scheme, B):
    """Per-sequence counts: one token, inside a page, a page boundary, inside
    the ring (KIVI) or near the end, the fill level; repeated over B."""
    from oracle import accounting
    q = accounting.flush_plan(T, R)[0] if scheme == synth.KIVI else T
    picks = [1, 45, 64 if T >= 64 else T, (q + T) // 2 if T > q else T - 1, T, max(1, q - 7)]
    return [min(T, max(1, picks[i % len(picks)])) for i in range(B)]


@pytest.mark.parametrize("scheme,bits,d,hg,dtype,R,T,rope,splits", CASES)
def test_ragged_decode(scheme, bits, d, hg, dtype, R, T, rope, splits):
    w = small(scheme, bits, d, dtype, R, B=6, hg=hg, T=T, rope=rope)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    lens = lengths(T, R, scheme, w.batch)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws, k_scale=ks, v_scale=vs)
    want = oc.decode(0, H.values(q), rope_theta=rope, seq_tokens=lens)
    err = H.max_err(out, want)
    assert err <= H.ATOL, (lens, err)


@pytest.mark.parametrize("case", [0, 2, 4, 11, 14, 9])
def test_ragged_full_lengths_match_uniform(case):
    """All counts at the fill level: the same bits as kvq_decode_attention."""
    scheme, bits, d, hg, dtype, R, T, rope, splits = CASES[case]
    w = small(scheme, bits, d, dtype, R, B=3, hg=hg, T=T, rope=rope)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    want = H.decode(cfg, cache, 0, T, q, ks, vs)
    seq = torch.full((w.batch,), T, dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws, k_scale=ks, v_scale=vs)
    assert torch.equal(out, want)


def test_ragged_counts_are_clamped():
    """Counts below 1 or above the fill level behave as 1 and the fill level."""
    scheme, bits, d, hg, dtype, R, T, rope, splits = CASES[0]
    w = small(scheme, bits, d, dtype, R, B=4, hg=hg, T=T, rope=rope)
    cfg, cache, oc, *_ = run_append(w, [T], capacity=T + 40)
    q = synth.query(w, device=DEV)
    raw = [0, -5, T + 100, 300]
    seq = torch.tensor(raw, dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws)
    want = oc.decode(0, H.values(q), seq_tokens=[1, 1, T, 300])
    assert H.max_err(out, want) <= H.ATOL
