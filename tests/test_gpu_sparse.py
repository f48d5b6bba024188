"""GPU parity of dense-and-sparse KIVI pages (one outlier per key channel and
per value token moved to an exact side matrix), through the C ABI.

Append: every defined byte of the cache -- dense codes, scales, offsets, the
side matrix's values and indices, ring rows -- equals the oracle's image for
several chunkings. Decode: outputs within max-abs 2e-3 of the oracle's fp64
attention over the dense-and-sparse dequantised cache, with and without the
rotary embedding, uniform, ragged and several queries per sequence. The inputs
carry isolated spikes (1 % of elements x 40) on top of the workloads' outlier
channels and tokens, so the side matrix holds values that matter."""

import numpy as np
import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"

CHUNKINGS = {
    "one": lambda T: [T],
    "steps": lambda T: [1] * 45 + [T - 45],
    "mixed": lambda T: [7, 32, 1, 100, 60, T - 200],
}


def sparse(bits, d, dtype=torch.bfloat16, R=0, B=2, Hkv=2, hg=2, T=300, rope=0.0, v_bits=0):
    return synth.Workload(f"sp{bits}d{d}", 60 + bits, synth.KIVI, bits, B, Hkv * hg, Hkv, d, T,
                          residual=R, in_dtype=dtype, q_dtype=dtype,
                          k_outlier_channels=min(4, d // 16), k_outlier_factor=20.0,
                          v_outlier_frac=0.01, v_outlier_factor=10.0, rope_theta=rope,
                          v_bits=v_bits, outliers=1, spike_frac=0.01, spike_factor=40.0)


def run(w, chunks, capacity):
    cfg = H.config(w, capacity)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, capacity)
    k, v = synth.keys_values(w, device=DEV)
    H.append_chunks(cfg, cache, k, v, chunks, oc=oc)
    torch.cuda.synchronize()
    return cfg, cache, oc, k, v


@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("bits,v_bits,d,dtype,R", [
    (2, 0, 128, torch.bfloat16, 128), (4, 0, 128, torch.bfloat16, 64),
    (8, 0, 64, torch.float32, 0), (4, 2, 256, torch.bfloat16, 37), (2, 0, 32, torch.float32, 5)])
def test_append_sparse_bytes(bits, v_bits, d, dtype, R, chunking):
    w = sparse(bits, d, dtype, R, v_bits=v_bits)
    cfg, cache, oc, *_ = run(w, CHUNKINGS[chunking](w.tokens), capacity=320)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"sparse b{bits} v{v_bits} d{d} {chunking}")


def test_append_sparse_ties_and_signed_zeros():
    """Vectors of equal magnitudes (+a/-a, zeros of both signs): the lower
    index moves, the sign of a moved zero is kept."""
    w = sparse(2, 64, torch.float32, 0, B=1, Hkv=1, hg=1, T=64)
    k = torch.randint(-2, 3, (1, 64, 1, 64), dtype=torch.float32)
    v = torch.randint(-2, 3, (1, 64, 1, 64), dtype=torch.float32)
    k[0, :32, 0, 5] = -0.0
    v[0, 40, 0, :] = 0.0
    v[0, 40, 0, ::2] = -0.0
    cfg = H.config(w, 64)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 64)
    H.append_chunks(cfg, cache, k.to(DEV).contiguous(), v.to(DEV).contiguous(), [64], oc=oc)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "sparse ties")


DECODE = [
    # bits, v_bits, d, hg, dtype, R, T, rope, splits
    (2, 0, 128, 4, torch.bfloat16, 128, 700, 0.0, 0),
    (4, 0, 128, 4, torch.bfloat16, 64, 555, 0.0, 3),
    (4, 2, 64, 2, torch.bfloat16, 20, 300, 0.0, 1),
    (8, 0, 256, 8, torch.bfloat16, 40, 300, 0.0, 2),
    (2, 0, 32, 1, torch.float32, 3, 98, 0.0, 0),
    (2, 0, 128, 4, torch.bfloat16, 128, 900, 500000.0, 0),   # rotary keys
    (4, 4, 64, 1, torch.float32, 0, 161, 10000.0, 4),
]


@pytest.mark.parametrize("bits,v_bits,d,hg,dtype,R,T,rope,splits", DECODE)
def test_decode_sparse(bits, v_bits, d, hg, dtype, R, T, rope, splits):
    w = sparse(bits, d, dtype, R, hg=hg, T=T, rope=rope, v_bits=v_bits)
    cfg, cache, oc, *_ = run(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q)
    want = oc.decode(0, H.values(q), rope_theta=rope)
    err = H.max_err(out, want)
    print(f"[sparse decode] b{bits} d{d} hg{hg} rope {rope}: max-abs error {err:.2e}", flush=True)
    assert err <= H.ATOL, err
    if bits > 2:
        return
    # the side matrix matters: the same tokens in plain 2-bit pages are further off
    plain = oc.__class__(synth.KIVI, bits, 1, w.batch, w.kv_heads, d, T + 40, residual=R,
                         in_dtype="bf16" if dtype == torch.bfloat16 else "f32",
                         v_bits=v_bits or None)
    plain.raw_k, plain.raw_v = oc.raw_k, oc.raw_v
    assert np.max(np.abs(plain.decode(0, H.values(q), rope_theta=rope) - want)) > 10 * H.ATOL


def test_decode_sparse_ragged_and_multi():
    """A ragged batch appended by per-sequence calls (each sequence its own
    page/ring split), decoded at its fill levels; and several causal queries
    per sequence on a uniform cache."""
    from oracle.cache import RaggedCache
    lens = [400, 150, 97]
    w = sparse(2, 128, torch.bfloat16, 64, B=3, hg=4, T=max(lens))
    cfg = H.config(w, 440)
    cache = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    rc = RaggedCache(synth.KIVI, 2, 1, 3, w.kv_heads, w.head_dim, 440, residual=64,
                     in_dtype="bf16", outliers=1)
    kn, vn = k.clone(), v.clone()
    for b, n in enumerate(lens):       # rows past each sequence's count are never read
        kn[b, n:] = float("nan")
        vn[b, n:] = float("nan")
        rc.append(0, b, H.host(k[b, :n]), H.host(v[b, :n]))
    zeros = torch.zeros(3, dtype=torch.int64, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kvq.kvq_quantize_append_ragged(cfg, cache, 0, zeros, seq, kn.contiguous(), vn.contiguous())
    want, mask = rc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "sparse ragged")
    q = synth.query(w, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, max(lens), device=DEV)
    kvq.kvq_decode_attention_ragged(cfg, cache, 0, max(lens), seq, q, out, ws)
    assert H.max_err(out, rc.decode(0, H.values(q))) <= H.ATOL

    wu = sparse(2, 128, torch.bfloat16, 64, B=3, hg=4, T=400)
    cfg, cache, oc, *_ = run(wu, [wu.tokens], capacity=440)
    nq = 5
    qm = torch.stack([synth.query(wu, device=DEV, tag=1 + i) for i in range(nq)], dim=1).contiguous()
    om = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
    wsm = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, wu.tokens, kvq.KVQ_BYTES_WORKSPACE),
                      dtype=torch.uint8, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, wu.tokens, qm, om, wsm)
    assert H.max_err(om, oc.decode_multi(0, H.values(qm))) <= H.ATOL
