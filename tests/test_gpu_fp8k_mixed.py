"""GPU parity of keys and values in different cache types: FP8 E4M3 keys
with the KV head's static key scale and per-token values at v_bits, either
symmetric (KVQ_FP8K_SYMV) or KIVI's asymmetric codes with a per-token scale
and offset (KVQ_FP8K_KIVIV), through the C ABI: every defined byte of the
cache equals the oracle's image for several chunkings; decode within max-abs
2e-3 of the oracle's fp64 attention over the dequantised cache (GQA 1-8,
split counts, rotary keys, several queries per sequence, ragged and paged
batches)."""

import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"

CHUNKINGS = {
    "one": lambda T: [T],
    "steps": lambda T: [1] * 40 + [T - 40],
    "mixed": lambda T: [7, 32, 1, 100, 60, T - 200],
}


SCHEMES = {"symv": synth.FP8K_SYMV, "kiviv": synth.FP8K_KIVIV}


def mixed(vb, d, dtype=torch.bfloat16, B=2, Hkv=2, hg=2, T=260, rope=0.0, scheme=synth.FP8K_SYMV):
    return synth.Workload(f"mx{scheme}v{vb}d{d}", 80 + vb + 10 * scheme, scheme, 8, B, Hkv * hg, Hkv, d, T,
                          in_dtype=dtype, q_dtype=dtype, k_outlier_channels=min(4, d // 16),
                          k_outlier_factor=20.0, v_outlier_frac=0.01, v_outlier_factor=10.0,
                          rope_theta=rope, v_bits=vb)


def run(w, chunks, capacity):
    cfg = H.config(w, capacity)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, capacity)
    k, v = synth.keys_values(w, device=DEV)
    ks, _ = synth.fp8_scales(k, v)
    ks = ks.to(DEV)
    H.append_chunks(cfg, cache, k, v, chunks, ks=ks, oc=oc)
    torch.cuda.synchronize()
    return cfg, cache, oc, k, v, ks


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("vb,d,dtype", [(2, 128, torch.bfloat16), (3, 64, torch.float32),
                                        (4, 32, torch.bfloat16), (8, 256, torch.float32)])
def test_append_bytes(vb, d, dtype, chunking, scheme):
    w = mixed(vb, d, dtype, scheme=SCHEMES[scheme])
    cfg, cache, oc, *_ = run(w, CHUNKINGS[chunking](w.tokens), capacity=288)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"fp8k_{scheme} v{vb} d{d} {chunking}")


DECODE = [
    # vb, d, hg, dtype, T, rope, splits
    (4, 128, 4, torch.bfloat16, 700, 0.0, 0),
    (2, 128, 8, torch.bfloat16, 333, 0.0, 3),
    (8, 64, 1, torch.float32, 97, 0.0, 1),
    (3, 64, 2, torch.bfloat16, 515, 10000.0, 0),
    (4, 256, 4, torch.float32, 300, 500000.0, 5),
    (2, 32, 2, torch.bfloat16, 64, 0.0, 0),
]


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("vb,d,hg,dtype,T,rope,splits", DECODE)
def test_decode(vb, d, hg, dtype, T, rope, splits, scheme):
    w = mixed(vb, d, dtype, hg=hg, T=T, rope=rope, scheme=SCHEMES[scheme])
    cfg, cache, oc, k, v, ks = run(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q, ks=ks)
    err = H.max_err(out, oc.decode(0, H.values(q), rope_theta=rope))
    print(f"[fp8k_{scheme} decode] v{vb} d{d} hg{hg} rope {rope}: max-abs error {err:.2e}", flush=True)
    assert err <= H.ATOL, err


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_decode_multi_and_ragged(scheme):
    from oracle.cache import RaggedCache
    w = mixed(4, 128, torch.bfloat16, B=3, hg=4, T=400, scheme=SCHEMES[scheme])
    cfg, cache, oc, k, v, ks = run(w, [w.tokens], capacity=440)
    nq = 5
    qm = torch.stack([synth.query(w, device=DEV, tag=1 + i) for i in range(nq)], dim=1).contiguous()
    om = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
    ws = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, w.tokens, kvq.KVQ_BYTES_WORKSPACE),
                     dtype=torch.uint8, device=DEV)
    kvq.kvq_decode_attention_multi(cfg, cache, 0, w.tokens, qm, om, ws, k_scale=ks)
    assert H.max_err(om, oc.decode_multi(0, H.values(qm))) <= H.ATOL
    assert int(ws.count_nonzero()) == 0

    lens = [400, 150, 33]
    cfg2 = H.config(w, 440)
    cache2 = kvq.alloc_cache(cfg2)
    rc = RaggedCache(SCHEMES[scheme], 8, 1, 3, w.kv_heads, w.head_dim, 440, in_dtype="bf16", v_bits=4)
    kn, vn = k.clone(), v.clone()
    for b, n in enumerate(lens):
        kn[b, n:] = float("nan")
        vn[b, n:] = float("nan")
        rc.append(0, b, H.host(k[b, :n]), H.host(v[b, :n]), H.host(ks))
    zeros = torch.zeros(3, dtype=torch.int64, device=DEV)
    seq = torch.tensor(lens, dtype=torch.int64, device=DEV)
    kvq.kvq_quantize_append_ragged(cfg2, cache2, 0, zeros, seq, kn.contiguous(), vn.contiguous(), k_scale=ks)
    want, mask = rc.cache_image()
    H.compare_bytes(cache2.cpu().numpy(), want, mask, f"fp8k_{scheme} ragged")
    q = synth.query(w, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws2 = kvq.alloc_workspace(cfg2, max(lens), device=DEV)
    kvq.kvq_decode_attention_ragged(cfg2, cache2, 0, max(lens), seq, q, out, ws2, k_scale=ks)
    assert H.max_err(out, rc.decode(0, H.values(q))) <= H.ATOL


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_paged(scheme):
    """A paged cache (block table over a shared pool) with FP8 keys and
    per-token values: bytes equal the oracle's paged image, decode equals the
    slab layout's bit for bit and the oracle within 2e-3."""
    import numpy as np
    from oracle.cache import RaggedCache, paged_image
    from test_gpu_ragged import B, CALLS, CAP, ragged_inputs
    T = max(sum(c[b] for c in CALLS) for b in range(B))
    w = mixed(2, 64, torch.bfloat16, B=B, hg=4, T=T, scheme=SCHEMES[scheme])
    cfg = H.config(w, CAP)
    pages = -(-CAP // 32)
    nb = B * pages + 5
    table_h = np.random.default_rng(7).permutation(nb)[:B * pages].astype(np.int32).reshape(B, pages)
    table = torch.from_numpy(table_h).to(DEV)
    paged = torch.zeros(kvq.kvq_paged_cache_bytes(cfg, nb), dtype=torch.uint8, device=DEV)
    slab = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    ks = synth.fp8_scales(k, v)[0].to(DEV)
    oc = RaggedCache(SCHEMES[scheme], 8, 1, B, w.kv_heads, w.head_dim, CAP, in_dtype="bf16", v_bits=2)
    past = [0] * B
    for counts in CALLS:
        kn, vn = ragged_inputs(w, k, v, past, counts)
        sp = torch.tensor(past, dtype=torch.int64, device=DEV)
        sn = torch.tensor(counts, dtype=torch.int64, device=DEV)
        kvq.kvq_quantize_append_paged(cfg, paged, 0, table, nb, sp, sn, kn, vn, ks, None)
        kvq.kvq_quantize_append_ragged(cfg, slab, 0, sp, sn, kn, vn, k_scale=ks)
        for b, n in enumerate(counts):
            oc.append(0, b, H.host(k[b, past[b]:past[b] + n]), H.host(v[b, past[b]:past[b] + n]), H.host(ks))
            past[b] += n
    torch.cuda.synchronize()
    want, mask = paged_image(oc, table_h, nb)
    H.compare_bytes(paged.cpu().numpy(), want, mask, f"fp8k_{scheme} paged")
    q = synth.query(w, device=DEV)
    seq = torch.tensor(past, dtype=torch.int64, device=DEV)
    out_p = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    out_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_paged(cfg, paged, 0, table, nb, T, seq, q, out_p, ws, k_scale=ks)
    kvq.kvq_decode_attention_ragged(cfg, slab, 0, T, seq, q, out_s, ws, k_scale=ks)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_s)
    assert H.max_err(out_p, oc.decode(0, H.values(q))) <= H.ATOL
