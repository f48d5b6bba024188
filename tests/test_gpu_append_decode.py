"""kvq_append_decode (one token appended, then decode) against the two calls
it stands for (kvq_quantize_append of one token, kvq_decode_attention), step
by step across page flushes: the same output and the same cache bytes, bit for
bit, on the fused one-launch path (KIVI matrix-core kernel, token into the
ring) and on the fallbacks (flush steps, rotary GQA-4, generic and FP8
kernels); and the final decode within 2e-3 of the oracle."""

import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth
from test_gpu_parity import small

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # scheme, bits, v_bits, d, hg, R, rope
    (synth.KIVI, 2, 0, 128, 4, 64, 0.0),        # fused (eight-wave matrix-core kernel)
    (synth.KIVI, 4, 2, 128, 4, 40, 0.0),        # fused, 4-bit keys / 2-bit values
    (synth.KIVI, 4, 0, 64, 2, 16, 0.0),         # fused (four-wave kernel)
    (synth.KIVI, 2, 0, 128, 2, 64, 500000.0),   # fused, rotary keys at GQA 2
    (synth.KIVI, 2, 0, 128, 4, 64, 500000.0),   # rotary GQA 4: append, then decode
    (synth.KIVI, 2, 0, 128, 4, 0, 0.0),         # R = 0: every 32nd step flushes its own token
    (synth.KIVI, 8, 0, 128, 4, 32, 0.0),        # generic kernel
    (synth.FP8_E4M3, 8, 0, 128, 4, 0, 0.0),     # FP8 pages
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}b{c[1]}v{c[2]}d{c[3]}g{c[4]}R{c[5]}r{int(c[6])}"
                                             for c in CASES])
def test_append_decode_matches_two_calls(case):
    scheme, bits, v_bits, d, hg, R, rope = case
    T0, steps = 250, 70
    w = small(scheme, bits, d, torch.bfloat16, R, B=3, hg=hg, T=T0 + steps, rope=rope, v_bits=v_bits)
    cfg = H.config(w, T0 + steps + 8)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if scheme == synth.FP8_E4M3:
        ks, vs = synth.fp8_scales(k, v)
    ca = kvq.alloc_cache(cfg)
    cb = kvq.alloc_cache(cfg)
    for c in (ca, cb):
        kvq.kvq_quantize_append(cfg, c, 0, 0, T0, k[:, :T0].contiguous(), v[:, :T0].contiguous(), ks, vs)
    q = synth.query(w, device=DEV)
    wa = kvq.alloc_workspace(cfg, device=DEV)
    wb = kvq.alloc_workspace(cfg, device=DEV)
    oa = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ob = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    for i in range(steps):
        t = T0 + i
        kn, vn = k[:, t:t + 1].contiguous(), v[:, t:t + 1].contiguous()
        kvq.kvq_append_decode(cfg, ca, 0, t, kn, vn, q, oa, wa, k_scale=ks, v_scale=vs)
        kvq.kvq_quantize_append(cfg, cb, 0, t, 1, kn, vn, ks, vs)
        kvq.kvq_decode_attention(cfg, cb, 0, t + 1, q, ob, wb, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (case, i)
    assert torch.equal(ca, cb)
    oc = H.oracle_cache(w, T0 + steps + 8)
    oc.append(0, H.host(k), H.host(v), None if ks is None else H.host(ks),
              None if vs is None else H.host(vs))
    assert H.max_err(oa, oc.decode(0, H.values(q), rope_theta=rope)) <= H.ATOL
