"""GPU parity of paged caches (block tables), through the C ABI: ragged
appends into a paged cache whose table scatters every sequence's pages over a
shared pool (a random permutation, plus unused blocks), on every append and
decode kernel (the case list of the ragged tests). The paged bytes equal the
oracle's paged image bit for bit; decode is within 2e-3 of the oracle and
bit-identical to the same calls on the slab layout."""

import numpy as np
import pytest
import torch

import harness as H
import kv_cache_quantisation_amd as kvq
import synth
from oracle.cache import RaggedCache, paged_image
from test_gpu_parity import small
from test_gpu_ragged import B, CALLS, CAP, CASES, ragged_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}b{c[1]}d{c[2]}g{c[3]}r{int(c[6])}"
                                             for c in CASES])
def test_paged_append_and_decode(case):
    scheme, bits, d, hg, dtype, R, rope, splits = case
    T = max(sum(c[b] for c in CALLS) for b in range(B))
    w = small(scheme, bits, d, dtype, R, B=B, hg=hg, T=T, rope=rope)
    cfg = H.config(w, CAP)
    cfg.num_splits = splits
    kvq.kvq_cache_bytes(cfg, CAP, kvq.KVQ_BYTES_CACHE)   # (validates the config)
    pages = (CAP - R) // 32 if scheme == synth.KIVI else -(-CAP // 32)
    nb = B * pages + 7
    perm = np.random.default_rng(scheme * 100 + bits * 10 + d).permutation(nb)
    table_h = perm[:B * pages].astype(np.int32).reshape(B, pages)
    table = torch.from_numpy(table_h).to(DEV)
    print(f"[paged] scheme {scheme} bits {bits} d {d} hg {hg} R {R} rope {rope}: "
          f"{pages} pages per sequence, {nb} blocks", flush=True)
    paged = torch.zeros(kvq.kvq_paged_cache_bytes(cfg, nb), dtype=torch.uint8, device=DEV)
    slab = kvq.alloc_cache(cfg)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if scheme in (synth.FP8_E4M3, synth.FP8_E5M2):
        fmax = 57344.0 if scheme == synth.FP8_E5M2 else 448.0
        ks, vs = (x.to(DEV) for x in synth.fp8_scales(k, v, fmax))
    oc = RaggedCache(w.scheme, w.bits, 1, w.batch, w.kv_heads, w.head_dim, CAP, residual=R,
                     in_dtype="bf16" if dtype == torch.bfloat16 else "f32")
    past = [0] * B
    for counts in CALLS:
        kn, vn = ragged_inputs(w, k, v, past, counts)
        sp = torch.tensor(past, dtype=torch.int64, device=DEV)
        sn = torch.tensor(counts, dtype=torch.int64, device=DEV)
        kvq.kvq_quantize_append_paged(cfg, paged, 0, table, nb, sp, sn, kn, vn, ks, vs)
        kvq.kvq_quantize_append_ragged(cfg, slab, 0, sp, sn, kn, vn, ks, vs)
        for b, n in enumerate(counts):
            oc.append(0, b, H.host(k[b, past[b]:past[b] + n]), H.host(v[b, past[b]:past[b] + n]),
                      None if ks is None else H.host(ks), None if vs is None else H.host(vs))
            past[b] += n
    torch.cuda.synchronize()
    want, mask = paged_image(oc, table_h, nb)
    H.compare_bytes(paged.cpu().numpy(), want, mask, f"paged scheme {scheme} b{bits} d{d}")
    q = synth.query(w, device=DEV)
    seq = torch.tensor(past, dtype=torch.int64, device=DEV)
    out_p = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    out_s = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, T, device=DEV)
    kvq.kvq_decode_attention_paged(cfg, paged, 0, table, nb, T, seq, q, out_p, ws, k_scale=ks,
                                   v_scale=vs)
    kvq.kvq_decode_attention_ragged(cfg, slab, 0, T, seq, q, out_s, ws, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_s)
    err = H.max_err(out_p, oc.decode(0, H.values(q), rope_theta=rope))
    assert err <= H.ATOL, err


def test_paged_sparse_pages():
    """Dense-and-sparse KIVI pages in a paged cache."""
    w = synth.Workload("pgsp", 55, synth.KIVI, 2, 2, 8, 2, 128, 300, residual=64,
                       k_outlier_channels=4, k_outlier_factor=20.0, v_outlier_frac=0.01,
                       v_outlier_factor=10.0, outliers=1, spike_frac=0.01, spike_factor=40.0)
    cfg = H.config(w, 320)
    pages = (320 - 64) // 32
    nb = 2 * pages + 1
    table_h = np.random.default_rng(1).permutation(nb)[:2 * pages].astype(np.int32).reshape(2, pages)
    table = torch.from_numpy(table_h).to(DEV)
    paged = torch.zeros(kvq.kvq_paged_cache_bytes(cfg, nb), dtype=torch.uint8, device=DEV)
    k, v = synth.keys_values(w, device=DEV)
    oc = RaggedCache(synth.KIVI, 2, 1, 2, 2, 128, 320, residual=64, in_dtype="bf16", outliers=1)
    zeros = torch.zeros(2, dtype=torch.int64, device=DEV)
    seq = torch.tensor([300, 300], dtype=torch.int64, device=DEV)
    kvq.kvq_quantize_append_paged(cfg, paged, 0, table, nb, zeros, seq, k, v)
    for b in range(2):
        oc.append(0, b, H.host(k[b]), H.host(v[b]))
    want, mask = paged_image(oc, table_h, nb)
    H.compare_bytes(paged.cpu().numpy(), want, mask, "paged sparse")
    q = synth.query(w, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = kvq.alloc_workspace(cfg, 300, device=DEV)
    kvq.kvq_decode_attention_paged(cfg, paged, 0, table, nb, 300, seq, q, out, ws)
    assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL
