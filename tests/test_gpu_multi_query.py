"""GPU parity of decode with several causal queries per sequence
(kvq_decode_attention_multi): query i at position T - n_q + i attends to
tokens [0, T - n_q + i] of the cache, compared with the oracle's decode_multi
(float64) on the same seeded inputs, for every scheme, with and without
rotary keys, queries whose tokens sit in KIVI's ring or in its pages (the
matrix-core kernel when the cache's inputs are 16-bit, one, two or four
queries per block; the generic kernel for fp32 inputs), and FP8 and bfloat16
caches (their matrix-core kernel without rotary keys)."""

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
    # scheme, bits, d, hg, dtype, R, T, rope, splits, n_q[, value bits, batch]
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 700, 0.0, 0, 4),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 300, 0.0, 0, 40),     # queries over pages
    (synth.KIVI, 4, 64, 2, torch.float32, 16, 257, 10000.0, 3, 17),
    (synth.KIVI, 2, 128, 2, torch.bfloat16, 128, 500, 500000.0, 0, 8),
    (synth.SYM_TOKEN, 4, 32, 1, torch.float32, 0, 200, 0.0, 0, 5),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 333, 0.0, 0, 3),
    (synth.FP8_E5M2, 8, 64, 2, torch.bfloat16, 0, 97, 500000.0, 2, 6),
    (synth.BF16_CACHE, 16, 128, 4, torch.bfloat16, 0, 333, 0.0, 0, 33),
    # KIVI 16-bit-input caches whose queries sit in the ring: matrix-core kernel
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 1000, 10000.0, 0, 3),   # rotary, GQA 4
    (synth.KIVI, 4, 128, 8, torch.bfloat16, 64, 450, 0.0, 0, 5),
    (synth.KIVI, 2, 64, 1, torch.bfloat16, 32, 200, 0.0, 1, 6),          # one split: no merge
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 32, 100, 0.0, 0, 36),        # n_q = ring tokens
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 90, 0.0, 0, 7),         # no pages yet
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 32, 100, 0.0, 0, 37),        # one more: in a page
    # GQA 4 without rotary keys, an even n_q in the ring: two queries per
    # block (key columns and value rows of both in one product)
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 64, 400, 0.0, 3, 6),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 900, 0.0, 1, 2),        # one split: no merge
    (synth.KIVI, 2, 64, 4, torch.bfloat16, 64, 333, 0.0, 5, 8),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 40, 1000, 0.0, 0, 40),       # n_q = ring tokens
    # queries whose tokens are in pages (chunks longer than the ring): each
    # row's last page masked after its own token
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 32, 300, 10000.0, 0, 70),    # rotary, GQA 4
    (synth.KIVI, 2, 64, 2, torch.bfloat16, 0, 150, 500000.0, 2, 40),     # rotary, GQA 2
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 32, 200, 0.0, 0, 100),
    (synth.KIVI, 2, 128, 8, torch.bfloat16, 128, 640, 0.0, 0, 300),
    # every token a query (the first sees token 0 alone): all in pages, all
    # in the ring, rotary
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 64, 0.0, 0, 64),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 50, 0.0, 0, 50),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 96, 10000.0, 0, 96),
    # two queries per block with their tokens in pages; the first query of
    # the first block sits at a page boundary (token 320), so the page after
    # holds none of its tokens (many splits: it is a wave's first page)
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 361, 0.0, 11, 42),
    (synth.KIVI, 4, 64, 4, torch.bfloat16, 8, 361, 0.0, 9, 42),
    # a block whose first query's token is the last quantised one (288) and
    # whose second is the first ring token: every page whole, one ring step
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 16, 305, 0.0, 0, 22),
    # four queries per block over dequantised keys (a multiple of four
    # queries, GQA 4, 2-bit values; value bits and batch last): the block's
    # first query's token in the last page and the other three in the ring
    # (each sees a different part of it)
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 16, 305, 0.0, 0, 20, 0, 26),
    # a block whose first query sees exactly ten pages: the page after holds
    # none of its tokens (weight 0), many splits
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 363, 0.0, 11, 44, 0, 12),
    # 4-bit keys with 2-bit values, head_dim 64 and 128, pages and ring
    (synth.KIVI, 4, 64, 4, torch.bfloat16, 8, 361, 0.0, 9, 44, 2, 12),
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 64, 500, 0.0, 0, 16, 2, 32),
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 32, 300, 0.0, 3, 100, 2, 6),
    (synth.KIVI, 4, 64, 4, torch.bfloat16, 16, 300, 0.0, 4, 8),           # 4-bit values too
    # long chunks (a multiple of 32 queries, batch x n_q / 32 x KV heads >=
    # 256): each chunk of 32 tokens copied and dequantised once per block of
    # 32 queries; early query groups end inside the pages, later ones reach
    # into the ring (a last ring chunk with rows past the last query), none
    # without a ring
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 32, 300, 0.0, 0, 128, 0, 32),
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 64, 400, 0.0, 0, 64, 2, 64),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 0, 256, 0.0, 0, 128, 0, 32),
    # FP8 and bfloat16 caches without rotary keys: their matrix-core kernel
    (synth.FP8_E5M2, 8, 128, 8, torch.bfloat16, 0, 301, 0.0, 3, 45),     # queries across pages
    # FP8 at GQA 4 with an even n_q: two queries per block (the second one's
    # columns and rows in the halves one query leaves idle); the open last
    # page in token rows; a first query at a page boundary whose partner's
    # token opens the next page (the first sees none of it); head_dim 64
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 333, 0.0, 0, 4),
    (synth.FP8_E5M2, 8, 128, 4, torch.bfloat16, 0, 321, 0.0, 3, 2),
    (synth.FP8_E4M3, 8, 64, 4, torch.bfloat16, 0, 200, 0.0, 5, 16),
    (synth.BF16_CACHE, 16, 128, 4, torch.bfloat16, 0, 150, 0.0, 2, 6),   # bfloat16 pages, two per block
    (synth.BF16_CACHE, 16, 64, 4, torch.bfloat16, 0, 129, 0.0, 0, 2),    # the second query opens a page
    (synth.BF16_CACHE, 16, 64, 2, torch.bfloat16, 0, 77, 0.0, 1, 9),     # one split: no merge
]


def queries(w, nq):
    return torch.stack([synth.query(w, device=DEV, tag=1 + i) for i in range(nq)], dim=1).contiguous()


@pytest.mark.parametrize("case", list(range(len(CASES))))
def test_multi_query_decode(case):
    scheme, bits, d, hg, dtype, R, T, rope, splits, nq = CASES[case][:10]
    vb = CASES[case][10] if len(CASES[case]) > 10 else 0
    batch = CASES[case][11] if len(CASES[case]) > 11 else 3
    w = small(scheme, bits, d, dtype, R, B=batch, hg=hg, T=T, rope=rope, v_bits=vb)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = queries(w, nq)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    one = kvq.kvq_cache_bytes(cfg, T, kvq.KVQ_BYTES_WORKSPACE)
    ws = torch.zeros(nq * one, dtype=torch.uint8, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, T, q, out, ws, k_scale=ks, v_scale=vs)
    want = oc.decode_multi(0, H.values(q), rope_theta=rope)
    err = H.max_err(out, want)
    assert err <= H.ATOL, err
    assert int(ws.count_nonzero()) == 0   # counters and partials


def test_single_query_is_the_plain_decode():
    scheme, bits, d, hg, dtype, R, T, rope, splits, nq = CASES[0]
    w = small(scheme, bits, d, dtype, R, B=3, hg=hg, T=T, rope=rope)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    q = synth.query(w, device=DEV)
    want = H.decode(cfg, cache, 0, T, q)
    out = torch.empty((w.batch, 1) + tuple(q.shape[1:]), dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, T, q.unsqueeze(1).contiguous(), out, ws)
    assert torch.equal(out[:, 0], want)




@pytest.mark.parametrize("nq", [4, 32])
@pytest.mark.parametrize("which", ["keys", "ring_keys", "queries"])
def test_four_query_blocks_f16_range(which, nq):
    """Four queries per block take the keys dequantised into f16 high and
    remainder parts and q' = q * sm_scale * log2(e) likewise; a page whose
    keys reach 2^15, or queries that do, are scaled by powers of two on the
    device and the scaling undone on the scores. Tokens X and Y of the first
    page are built so that X wins the softmax by more than 1e4 log2 units
    with the true operands, while Y would win had the large operand
    saturated at the f16 maximum (high and remainder parts both at 65504):
    "keys": X's channel 0 is 3e5 against q_0 = 1 (true score 3.8e4, 1.7e4
    saturated) and Y's channel 1 is 2e4 against q_1 = 9.8 (2.5e4);
    "queries": q_5 = 2e6 against X's channel 5 of 10 (q'_5 = 2.5e5, 1.3e5
    saturated) and q_6 = 3.9e5 against Y's channel 6 of 40; "ring_keys": as
    "keys" with X and Y residual tokens (keys rescaled per 32-token chunk of
    the ring by the long-chunk kernel). Every output row is then X's value
    row; plain 2e-3 against the oracle. n_q = 4: four queries per block;
    n_q = 32 over 256 sequences: the long-chunk kernel (32 per block)."""
    B = 2 if nq == 4 else 256
    w = small(synth.KIVI, 2, 128, torch.bfloat16, 16, B=B, Hkv=1, hg=4, T=100)
    T = w.tokens
    X, Y = (66, 67) if which == "ring_keys" else (3, 17)   # ring from token 64; queries from 68
    k, v = synth.keys_values(w, device=DEV)
    q = queries(w, nq).float()
    k = k.float()
    if which in ("keys", "ring_keys"):
        k[:, X, :, 0] = 3.0e5
        k[:, Y, :, 1] = 2.0e4
        q[:, :, :, 0] = 1.0
        q[:, :, :, 1] = 9.8
    else:
        k[:, :, :, 5:7] *= 0.1
        k[:, X, :, 5] = 10.0
        k[:, Y, :, 6] = 40.0
        q[:, :, :, 5] = 2.0e6
        q[:, :, :, 6] = 3.92e5
    k = k.to(torch.bfloat16).contiguous()
    q = q.to(torch.bfloat16).contiguous()
    cfg = H.config(w, T + 40)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, T + 40)
    H.append_chunks(cfg, cache, k, v, [T], oc=oc)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, T, kvq.KVQ_BYTES_WORKSPACE), dtype=torch.uint8, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, T, q, out, ws)
    want = oc.decode_multi(0, H.values(q))
    # the construction: every row is X's value row
    vx = want[:, :1, :1]
    assert np.allclose(want, np.broadcast_to(vx, want.shape), atol=1e-6)
    err = H.max_err(out, want)
    print(f"[four-query range] {which} n_q {nq}: max-abs error {err:.2e}", flush=True)
    assert err <= H.ATOL, err
