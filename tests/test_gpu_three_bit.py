"""GPU parity of 3-bit codes (fields straddle bytes and words), through the C
ABI: KIVI keys and/or values at 3 bits and the symmetric per-token scheme at 3
bits ("Quantising the Cache.", Twice the users for nearly nothing: the 3-bit
cache; KVQuant Key points: 3-bit keys and values). Cache bytes bit-exact
against the oracle for several chunkings; decode within 2e-3 of the oracle."""

import pytest
import torch

import harness as H
import synth
from test_gpu_parity import CHUNKINGS, run_append, small

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("bits,v_bits,d,dtype,R", [
    (3, 0, 128, torch.bfloat16, 128), (3, 0, 32, torch.float32, 5), (3, 2, 64, torch.bfloat16, 0),
    (4, 3, 128, torch.float32, 37), (8, 3, 256, torch.bfloat16, 16)])
def test_append_kivi_three_bit_bytes(bits, v_bits, d, dtype, R, chunking):
    w = small(synth.KIVI, bits, d, dtype, R, v_bits=v_bits)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=320)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"kivi k{bits} v{v_bits or bits} d{d} {chunking}")


@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("d,dtype", [(32, torch.float32), (128, torch.bfloat16), (64, torch.float32)])
def test_append_sym_three_bit_bytes(d, dtype, chunking):
    w = small(synth.SYM_TOKEN, 3, d, dtype, T=269)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=300)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"sym b3 d{d} {chunking}")


DECODE = [
    # scheme, bits, v_bits, d, hg, dtype, R, T, rope, splits
    (synth.KIVI, 3, 0, 128, 4, torch.bfloat16, 128, 700, 0.0, 0),
    (synth.KIVI, 3, 0, 32, 1, torch.float32, 3, 98, 0.0, 0),
    (synth.KIVI, 3, 2, 64, 2, torch.bfloat16, 20, 300, 0.0, 3),
    (synth.KIVI, 4, 3, 128, 8, torch.bfloat16, 40, 333, 0.0, 2),
    (synth.KIVI, 8, 3, 256, 2, torch.float32, 16, 257, 0.0, 0),
    (synth.KIVI, 3, 0, 128, 4, torch.bfloat16, 128, 900, 500000.0, 0),
    (synth.SYM_TOKEN, 3, 0, 32, 1, torch.float32, 0, 512, 0.0, 0),
    (synth.SYM_TOKEN, 3, 0, 128, 4, torch.bfloat16, 0, 300, 500000.0, 5),
]


@pytest.mark.parametrize("scheme,bits,v_bits,d,hg,dtype,R,T,rope,splits", DECODE)
def test_decode_three_bit(scheme, bits, v_bits, d, hg, dtype, R, T, rope, splits):
    w = small(scheme, bits, d, dtype, R, hg=hg, T=T, rope=rope, v_bits=v_bits)
    cfg, cache, oc, *_ = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q)
    err = H.max_err(out, oc.decode(0, H.values(q), rope_theta=rope))
    print(f"[3-bit decode] scheme {scheme} k{bits} v{v_bits or bits} d{d}: {err:.2e}", flush=True)
    assert err <= H.ATOL, err


def test_three_bit_sparse():
    """3-bit keys and values with one outlier per vector (KVQuant's nuq3 with
    outliers, here with uniform levels)."""
    w = synth.Workload("s3", 93, synth.KIVI, 3, 2, 8, 2, 128, 500, residual=64,
                       k_outlier_channels=4, k_outlier_factor=20.0, v_outlier_frac=0.01,
                       v_outlier_factor=10.0, outliers=1, spike_frac=0.01, spike_factor=40.0)
    cfg, cache, oc, *_ = run_append(w, [200, 1, 299], capacity=520)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "sparse 3-bit")
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, 500, q)
    assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL
