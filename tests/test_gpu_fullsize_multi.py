"""Several causal queries per sequence (kvq_decode_attention_multi) at full
workload sizes, in the launch configuration the benchmark times (automatic
split plan): query i of n_q, at position T - n_q + i, attends to tokens
[0, T - n_q + i] of the cache. Sampled (sequence, KV head) units are checked
against the oracle's fp64 attention over that unit's dequantised keys and
values (the KIVI page/ring split of the whole cache), cut at each query's own
token. KIVI caches run on their matrix-core kernels (four or 32 queries per
block for 8 and 64 queries), FP8 on its matrix-core kernel (two queries per
block for an even n_q)."""

import numpy as np
import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"

# case -> (workload, queries per sequence, (sequence, KV head) units checked)
# (kivi2 with 8 queries: four queries per block, their rows filling the chip)
CASES = {
    "kivi2": ("kivi2", 4, [(0, 0), (15, 7)]),
    "kivi2_8q": ("kivi2", 8, [(0, 0), (9, 3), (15, 7)]),
    "kivi2_64q": ("kivi2", 64, [(0, 0), (15, 7)]),
    "int4": ("int4", 8, [(31, 7)]),
    "longctx": ("longctx", 4, [(0, 3)]),
    "fp8": ("fp8", 3, [(63, 2)]),
    "fp8_4q": ("fp8", 4, [(0, 0), (63, 2)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_multi_query(name):
    wname, nq, units = CASES[name]
    w = synth.WORKLOADS[wname]
    T = w.tokens
    print(f"[fullsize-multi] {name}: B={w.batch} Hkv={w.kv_heads} d={w.head_dim} T={T} n_q={nq}",
          flush=True)
    cfg = H.config(w, T)
    cache = kvq.alloc_cache(cfg, zero=False)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if w.scheme == synth.FP8_E4M3:
        ks, vs = synth.fp8_scales(k, v)
    kvq.kvq_quantize_append(cfg, cache, 0, 0, T, k, v, ks, vs)
    qm = torch.stack([synth.query(w, device=DEV, tag=1 + i) for i in range(nq)], dim=1).contiguous()
    out = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, T, kvq.KVQ_BYTES_WORKSPACE),
                     dtype=torch.uint8, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, T, qm, out, ws, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0   # counters and partials

    hg = w.q_heads // w.kv_heads
    qv = H.values(qm)
    outh = out.cpu().numpy()
    assert np.isfinite(outh).all()
    for b, h in units:
        kf, vf = H.values(k[b, :, h]), H.values(v[b, :, h])
        ksh = None if ks is None else float(ks[h])
        vsh = None if vs is None else float(vs[h])
        kh, vh = H.oracle_dequant_head(w, kf, vf, T, ksh, vsh)
        worst = 0.0
        for i in range(nq):
            Ti = T - nq + i + 1
            want = H.oracle_attend_head(w, qv[b, i, h * hg:(h + 1) * hg], kh[:Ti], vh[:Ti], Ti)
            err = float(np.max(np.abs(outh[b, i, h * hg:(h + 1) * hg].astype(np.float64) - want)))
            worst = max(worst, err)
            assert err <= H.ATOL, (name, b, h, i, err)
        print(f"[fullsize-multi] {name} unit ({b},{h}): {nq} queries, max-abs error {worst:.2e}",
              flush=True)
