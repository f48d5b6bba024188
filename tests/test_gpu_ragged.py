"""GPU parity of the ragged-batch path: per-sequence quantize-append
(kvq_quantize_append_ragged), where every sequence keeps its own fill level,
and decode over those fill levels (kvq_decode_attention_ragged). The oracle is
RaggedCache (one single-sequence cache per sequence). Cache bytes must match
bit for bit in every defined field, decode within 2e-3 of the float64 oracle,
on every append and decode kernel."""

import numpy as np
import pytest
import torch

import kv_cache_quantisation_amd as kvq
import synth
import harness as H
from oracle.cache import RaggedCache
from test_gpu_parity import small

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)

CASES = [
    # scheme, bits, d, hg, dtype, R, rope, splits
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 0.0, 0),      # 8-wave matrix-core decode
    (synth.KIVI, 2, 64, 2, torch.float32, 0, 0.0, 5),
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 128, 0.0, 3),      # 4-wave matrix-core decode
    (synth.KIVI, 2, 128, 8, torch.bfloat16, 40, 0.0, 0),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 500000.0, 0),  # rotary, GQA 4
    (synth.KIVI, 2, 128, 2, torch.bfloat16, 40, 500000.0, 5),  # rotary, other GQA
    (synth.KIVI, 8, 128, 8, torch.bfloat16, 16, 0.0, 0),       # generic decode
    (synth.KIVI, 4, 32, 1, torch.float32, 3, 0.0, 0),
    (synth.KIVI, 4, 64, 2, torch.bfloat16, 20, 10000.0, 4),
    (synth.SYM_TOKEN, 4, 32, 1, torch.float32, 0, 0.0, 0),
    (synth.SYM_TOKEN, 2, 256, 2, torch.bfloat16, 0, 500000.0, 3),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 0.0, 0),    # FP8 pages
    (synth.FP8_E5M2, 8, 64, 2, torch.bfloat16, 0, 0.0, 3),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 500000.0, 0),
    (synth.BF16_CACHE, 16, 128, 4, torch.bfloat16, 0, 0.0, 0),  # bfloat16 pages
    (synth.BF16_CACHE, 16, 256, 2, torch.bfloat16, 0, 500000.0, 3),
]

B = 5
# per call, tokens appended by each sequence (0 = sequence skips the call):
# sequences end at 1, mid-page, in the KIVI ring, on flush boundaries, long
CALLS = [[1, 40, 300, 160, 0], [0, 7, 1, 32, 500], [0, 0, 45, 1, 129]]
CAP = 700


def ragged_inputs(w, k, v, past, counts):
    """[B, new_max, H, d] inputs of one call: sequence b's rows past_b ..
    past_b + n_b - 1 of its history, the unused rows NaN (never read)."""
    nmax = max(counts)
    shape = (w.batch, nmax, w.kv_heads, w.head_dim)
    kn = torch.full(shape, float("nan"), dtype=k.dtype, device=DEV)
    vn = torch.full(shape, float("nan"), dtype=v.dtype, device=DEV)
    for b, n in enumerate(counts):
        kn[b, :n] = k[b, past[b]:past[b] + n]
        vn[b, :n] = v[b, past[b]:past[b] + n]
    return kn, vn


def build(case, calls=CALLS):
    scheme, bits, d, hg, dtype, R, rope, splits = case
    T = max(sum(c[b] for c in calls) for b in range(B))       # longest history
    assert T <= CAP
    w = small(scheme, bits, d, dtype, R, B=B, hg=hg, T=T, rope=rope)
    cfg = H.config(w, CAP)
    cfg.num_splits = splits
    cache = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if scheme in (synth.FP8_E4M3, synth.FP8_E5M2):
        fmax = 57344.0 if scheme == synth.FP8_E5M2 else 448.0
        ks, vs = (x.to(DEV) for x in synth.fp8_scales(k, v, fmax))
    oc = RaggedCache(w.scheme, w.bits, 1, w.batch, w.kv_heads, w.head_dim, CAP, residual=R,
                     in_dtype="bf16" if dtype == torch.bfloat16 else "f32")
    past = [0] * B
    for counts in calls:
        kn, vn = ragged_inputs(w, k, v, past, counts)
        sp = torch.tensor(past, dtype=torch.int64, device=DEV)
        sn = torch.tensor(counts, dtype=torch.int64, device=DEV)
        kvq.kvq_quantize_append_ragged(cfg, cache, 0, sp, sn, kn, vn, ks, vs)
        for b, n in enumerate(counts):
            oc.append(0, b, H.host(k[b, past[b]:past[b] + n]), H.host(v[b, past[b]:past[b] + n]),
                      None if ks is None else ks.cpu().numpy(), None if vs is None else vs.cpu().numpy())
            past[b] += n
    torch.cuda.synchronize()
    return w, cfg, cache, oc, past, ks, vs


@pytest.mark.parametrize("case", list(range(len(CASES))))
def test_ragged_append_bytes_and_decode(case):
    w, cfg, cache, oc, fill, ks, vs = build(CASES[case])
    assert oc.tokens(0) == fill
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"ragged case {case}")
    q = synth.query(w, device=DEV)
    T = max(fill)
    seq = torch.tensor(fill, dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws, k_scale=ks, v_scale=vs)
    err = H.max_err(out, oc.decode(0, H.values(q), rope_theta=CASES[case][6]))
    assert err <= H.ATOL, (fill, err)


@pytest.mark.parametrize("case", [0, 2, 9, 11, 14])
def test_ragged_equal_counts_match_uniform_calls(case):
    """Equal counts for every sequence: the same bytes as kvq_quantize_append
    and the same decode output as kvq_decode_attention, bit for bit."""
    scheme, bits, d, hg, dtype, R, rope, splits = CASES[case]
    calls = [[37] * B, [0] * B, [1] * B, [200] * B]
    w, cfg, cache, oc, fill, ks, vs = build(CASES[case], calls)
    ref = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    H.append_chunks(cfg, ref, k, v, [37, 1, 200], ks=ks, vs=vs)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref)
    T = fill[0]
    q = synth.query(w, device=DEV)
    want = H.decode(cfg, ref, 0, T, q, ks, vs)
    seq = torch.full((w.batch,), T, dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws, k_scale=ks, v_scale=vs)
    assert torch.equal(out, want)


def test_ragged_counts_are_clamped():
    """Appended counts above the call's row bound act as the bound, negative
    ones as 0; decode counts above `tokens` act as `tokens`."""
    case = CASES[9]                                   # SYM 4-bit, d 32
    scheme, bits, d, hg, dtype, R, rope, splits = case
    w = small(scheme, bits, d, dtype, R, B=B, hg=hg, T=120, rope=rope)
    cfg = H.config(w, CAP)
    cache = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    kn, vn = k[:, :60].contiguous(), v[:, :60].contiguous()
    sp = torch.zeros(B, dtype=torch.int64, device=DEV)
    sn = torch.tensor([60, 500, -3, 10, 60], dtype=torch.int64, device=DEV)
    kvq.kvq_quantize_append_ragged(cfg, cache, 0, sp, sn, kn, vn)
    oc = RaggedCache(scheme, bits, 1, B, w.kv_heads, d, CAP, in_dtype="f32")
    for b, n in enumerate([60, 60, 0, 10, 60]):
        oc.append(0, b, H.host(k[b, :n]), H.host(v[b, :n]))
    torch.cuda.synchronize()
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "clamped counts")
    q = synth.query(w, device=DEV)
    seq = torch.tensor([60, 999, 1, 10, 60], dtype=torch.int64, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, 60, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, 60, seq, q, out, ws)
    got = out.cpu().numpy()
    qv = H.values(q)
    for b in (0, 1, 3, 4):                            # sequence 2 holds no token
        want_b = oc.seqs[b].decode(0, qv[b:b + 1])[0]
        assert np.max(np.abs(got[b] - want_b)) <= H.ATOL, b
