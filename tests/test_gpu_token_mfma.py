"""GPU parity of the matrix-core decode of caches whose codes carry a scale
per token: symmetric 2/4/8-bit keys and values (KVQ_SYM_TOKEN) and FP8 E4M3
keys with symmetric or KIVI 2/4/8-bit values (KVQ_FP8K_SYMV, KVQ_FP8K_KIVIV), at
head_dim 32-256 without rotary keys (`paged_mfma_kernel`; at head_dim 32 also
FP8 and bfloat16 pages): outputs within
max-abs 2e-3 of the oracle's fp64 attention over the dequantised cache, for
every GQA width, partial last pages (down to one token), split counts,
several queries per sequence and a ragged batch."""

import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth
from test_gpu_parity import run_append, small

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)

CASES = [
    # scheme, bits, v_bits, d, hg, dtype, T, splits
    (synth.SYM_TOKEN, 2, 0, 128, 4, torch.bfloat16, 700, 0),
    (synth.SYM_TOKEN, 4, 0, 128, 8, torch.bfloat16, 333, 3),
    (synth.SYM_TOKEN, 2, 0, 64, 1, torch.float32, 1, 0),
    (synth.SYM_TOKEN, 4, 0, 64, 2, torch.float32, 97, 1),
    (synth.SYM_TOKEN, 4, 0, 256, 4, torch.bfloat16, 260, 0),
    (synth.SYM_TOKEN, 2, 0, 256, 2, torch.bfloat16, 64, 5),
    (synth.FP8K_SYMV, 8, 2, 128, 4, torch.bfloat16, 515, 0),
    (synth.FP8K_SYMV, 8, 4, 64, 8, torch.float32, 31, 2),
    (synth.FP8K_SYMV, 8, 4, 256, 1, torch.bfloat16, 129, 0),
    (synth.FP8K_KIVIV, 8, 2, 64, 2, torch.bfloat16, 200, 0),
    (synth.FP8K_KIVIV, 8, 4, 128, 4, torch.bfloat16, 1000, 4),
    (synth.FP8K_KIVIV, 8, 2, 256, 8, torch.float32, 33, 1),
    # 8-bit codes (bytes converted as integers, channel/token order kept)
    (synth.SYM_TOKEN, 8, 0, 128, 4, torch.bfloat16, 300, 0),
    (synth.SYM_TOKEN, 8, 0, 64, 2, torch.float32, 45, 2),
    (synth.FP8K_SYMV, 8, 8, 128, 2, torch.bfloat16, 257, 0),
    (synth.FP8K_SYMV, 8, 0, 64, 4, torch.bfloat16, 7, 1),
    (synth.FP8K_KIVIV, 8, 8, 256, 4, torch.float32, 100, 3),
    # head_dim 32 (the tiny workload's shape first), FP8 and bfloat16 pages too
    (synth.SYM_TOKEN, 4, 0, 32, 1, torch.float32, 512, 0),
    (synth.SYM_TOKEN, 8, 0, 32, 4, torch.bfloat16, 70, 2),
    (synth.FP8K_KIVIV, 8, 4, 32, 2, torch.bfloat16, 65, 0),
    (synth.FP8K_SYMV, 8, 2, 32, 8, torch.float32, 200, 3),
    (synth.FP8_E4M3, 8, 0, 32, 4, torch.bfloat16, 333, 0),
    (synth.FP8_E5M2, 8, 0, 32, 2, torch.float32, 47, 1),
    (synth.BF16_CACHE, 16, 0, 32, 4, torch.bfloat16, 129, 0),
]


def build(case, B=2):
    scheme, bits, vb, d, hg, dtype, T, splits = case
    w = small(scheme, bits, d, dtype, B=B, hg=hg, T=T, v_bits=vb)
    if scheme in (synth.SYM_TOKEN, synth.FP8_E4M3, synth.FP8_E5M2, synth.BF16_CACHE):
        cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    else:
        from test_gpu_fp8k_mixed import run
        cfg, cache, oc, k, v, ks = run(w, [T], capacity=T + 40)
        vs = None
    cfg.num_splits = splits
    return w, cfg, cache, oc, ks, vs


@pytest.mark.parametrize("case", list(range(len(CASES))))
def test_decode(case):
    w, cfg, cache, oc, ks, vs = build(CASES[case])
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, w.tokens, q, ks, vs)
    err = H.max_err(out, oc.decode(0, H.values(q)))
    assert err <= H.ATOL, (case, err)


@pytest.mark.parametrize("nq", [5, 6])
@pytest.mark.parametrize("case", [0, 4, 6, 7, 10, 12, 14, 15, 17, 18, 19, 21])
def test_multi_query(case, nq):
    """Several queries; an even n_q at GQA 4 runs two queries per block."""
    w, cfg, cache, oc, ks, vs = build(CASES[case], B=3)
    nq = min(nq, w.tokens)
    q = torch.stack([synth.query(w, device=DEV, tag=1 + i) for i in range(nq)], dim=1).contiguous()
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, w.tokens, kvq.KVQ_BYTES_WORKSPACE), dtype=torch.uint8,
                     device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, w.tokens, q, out, ws, k_scale=ks, v_scale=vs)
    assert H.max_err(out, oc.decode_multi(0, H.values(q))) <= H.ATOL
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("case", [1, 6, 11, 13, 16, 18, 20, 21, 22, 23])
def test_ragged(case):
    """A ragged batch: each sequence appended to its own fill level (one
    ragged append), then decoded over its own tokens."""
    from oracle.cache import RaggedCache
    scheme, bits, vb, d, hg, dtype, T, splits = CASES[case]
    w = small(scheme, bits, d, dtype, B=3, hg=hg, T=T, v_bits=vb)
    lens = [T, max(1, T // 2), max(1, T // 3 + 1)]
    cfg = H.config(w, T + 40)
    cfg.num_splits = splits
    cache = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if scheme in (synth.FP8_E4M3, synth.FP8_E5M2):
        ks, vs = (x.to(DEV) for x in synth.fp8_scales(k, v, 57344.0 if scheme == synth.FP8_E5M2 else 448.0))
    elif scheme in (synth.FP8K_SYMV, synth.FP8K_KIVIV):
        ks = synth.fp8_scales(k, v)[0].to(DEV)
    rc = RaggedCache(scheme, bits, 1, 3, w.kv_heads, d, T + 40,
                     in_dtype="bf16" if dtype == torch.bfloat16 else "f32", v_bits=vb or None)
    kn, vn = k.clone(), v.clone()
    for b, n in enumerate(lens):
        kn[b, n:] = float("nan")   # never read
        vn[b, n:] = float("nan")
        rc.append(0, b, H.host(k[b, :n]), H.host(v[b, :n]), None if ks is None else H.host(ks),
                  None if vs is None else H.host(vs))
    zeros = torch.zeros(3, dtype=torch.int64, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kvq.kvq_quantize_append_ragged(cfg, cache, 0, zeros, seq, kn.contiguous(), vn.contiguous(), ks, vs)
    want, mask = rc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"token case {case} ragged")
    q = synth.query(w, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, T, seq, q, out, ws, k_scale=ks, v_scale=vs)
    assert H.max_err(out, rc.decode(0, H.values(q))) <= H.ATOL
