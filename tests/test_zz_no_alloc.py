"""The decode entry point that allocates nothing (kvq_decode_attention_noalloc)
against kvq_decode_attention with a workspace, through the C ABI.

Both run the same kernels with the same split plan, so their outputs must agree
bit for bit; both are also within 2e-3 of the oracle. Two calls in a row, the
second on a smaller cache, check that the shared scratch array (which keeps the
previous call's contents) is reused correctly; the configurations use several
splits per (sequence, KV head), so the arrival counters and the cross-block
merge are exercised."""

import numpy as np
import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def workload(scheme, bits, B, T, R, hg=4, Hkv=2, d=128, rope=0.0):
    return synth.Workload(f"na{scheme}b{bits}", 70 + bits, scheme, bits, B, Hkv * hg, Hkv, d, T,
                          residual=R, k_outlier_channels=4, k_outlier_factor=20.0,
                          v_outlier_frac=0.01, v_outlier_factor=10.0, rope_theta=rope)


def filled(w, splits=0):
    cfg = H.config(w, w.tokens, num_splits=splits)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, w.tokens)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if w.scheme == synth.FP8_E4M3:
        ks, vs = synth.fp8_scales(k, v)
    H.append_chunks(cfg, cache, k, v, [w.tokens], ks=ks, vs=vs, oc=oc)
    return cfg, cache, oc, ks, vs


CASES = [
    # (first call, second smaller call)
    (workload(synth.KIVI, 2, 4, 2000, 128), workload(synth.KIVI, 2, 2, 700, 128)),
    (workload(synth.KIVI, 4, 3, 1500, 64), workload(synth.FP8_E4M3, 8, 2, 900, 0)),
    (workload(synth.KIVI, 2, 2, 3000, 128, rope=500000.0), workload(synth.KIVI, 2, 1, 400, 32)),
]


@pytest.mark.parametrize("first,second", CASES, ids=["kivi2", "kivi4-fp8", "rope-kivi2"])
def test_noalloc_matches_workspace_decode(first, second):
    for w in (first, second):
        print(f"[noalloc] scheme {w.scheme} bits {w.bits} B={w.batch} T={w.tokens} "
              f"rope={w.rope_theta}", flush=True)
        cfg, cache, oc, ks, vs = filled(w)
        need = kvq.kvq_cache_bytes(cfg, w.tokens, kvq.KVQ_BYTES_WORKSPACE)
        assert need <= kvq.KVQ_NOALLOC_SCRATCH_BYTES
        counters = -(-w.batch * w.kv_heads * 4 // 256) * 256
        splits = (need - counters) // (w.batch * w.q_heads * (w.head_dim + 2) * 4)
        print(f"[noalloc] workspace {need} B, {splits} splits per (sequence, KV head)", flush=True)
        if w is first:
            assert splits >= 2     # the counters and the cross-block merge take part
        q = synth.query(w, device=DEV)
        want = H.decode(cfg, cache, 0, w.tokens, q, ks, vs)
        got = torch.full_like(want, float("nan"))
        kvq.kvq_decode_attention_noalloc(cfg, cache, 0, w.tokens, q, got, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        ref = oc.decode(0, H.values(q), rope_theta=w.rope_theta)
        assert H.max_err(got, ref) <= H.ATOL
        # again on the same array (the counters must have returned to zero)
        got2 = torch.full_like(want, float("nan"))
        kvq.kvq_decode_attention_noalloc(cfg, cache, 0, w.tokens, q, got2, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        assert torch.equal(got2, want)


def test_noalloc_rejects_sizes_beyond_the_array():
    w = workload(synth.KIVI, 2, 4096, 1 << 16, 128)
    cfg = H.config(w, w.tokens, num_splits=64)
    assert kvq.kvq_cache_bytes(cfg, w.tokens, kvq.KVQ_BYTES_WORKSPACE) > \
        kvq.KVQ_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(16, dtype=torch.uint8, device=DEV)
    st = kvq.kvq_decode_attention_noalloc(cfg, q, 0, w.tokens, q, q, check=False)
    assert st == kvq.KVQ_ERR_WORKSPACE
