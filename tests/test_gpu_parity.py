"""GPU parity of the HIP library against the oracle, through the C ABI.

Append: every defined bit of the cache (codes, scales, offsets, ring rows) must
equal the oracle's byte image -- bit-exact -- for several chunkings of the same
tokens. Decode: outputs within max-abs 2e-3 of the oracle's fp64 attention
over the dequantised cache."""

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


def small(scheme, bits, d, dtype=torch.bfloat16, R=0, B=2, Hkv=2, hg=2, T=300, rope=0.0,
          v_frac=0.01, v_bits=0):
    return synth.Workload(f"s{scheme}b{bits}d{d}", 90 + scheme * 10 + bits, scheme, bits, B,
                          Hkv * hg, Hkv, d, T, residual=R, in_dtype=dtype, q_dtype=dtype,
                          k_outlier_channels=min(4, d // 16), k_outlier_factor=20.0,
                          v_outlier_frac=v_frac, v_outlier_factor=10.0, rope_theta=rope,
                          v_bits=v_bits)


def run_append(w, chunks, capacity, scales=None):
    cfg = H.config(w, capacity)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, capacity)
    k, v = synth.keys_values(w, device=DEV)
    ks = vs = None
    if w.scheme in (synth.FP8_E4M3, synth.FP8_E5M2):
        fmax = 57344.0 if w.scheme == synth.FP8_E5M2 else 448.0
        ks, vs = scales if scales is not None else synth.fp8_scales(k, v, fmax)
        ks, vs = ks.to(DEV), vs.to(DEV)
    H.append_chunks(cfg, cache, k, v, chunks, ks=ks, vs=vs, oc=oc)
    torch.cuda.synchronize()
    return cfg, cache, oc, k, v, ks, vs


@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("bits,d,dtype,R", [
    (2, 128, torch.bfloat16, 128), (4, 128, torch.bfloat16, 128), (8, 128, torch.bfloat16, 128),
    (2, 32, torch.float32, 5), (4, 64, torch.float32, 0), (8, 256, torch.bfloat16, 37),
    (2, 256, torch.float32, 64), (4, 32, torch.bfloat16, 1)])
def test_append_kivi_bytes(bits, d, dtype, R, chunking):
    w = small(synth.KIVI, bits, d, dtype, R)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=320)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"kivi b{bits} d{d} R{R} {chunking}")


@pytest.mark.parametrize("chunking", list(CHUNKINGS))
@pytest.mark.parametrize("bits,v_bits,d,dtype,R", [
    (4, 2, 128, torch.bfloat16, 128), (8, 4, 64, torch.float32, 0), (8, 2, 256, torch.bfloat16, 37),
    (4, 2, 32, torch.bfloat16, 1), (8, 4, 128, torch.bfloat16, 5)])
def test_append_kivi_value_bits_bytes(bits, v_bits, d, dtype, R, chunking):
    """KIVI pages with value codes narrower than key codes, bit-exact."""
    w = small(synth.KIVI, bits, d, dtype, R, v_bits=v_bits)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=320)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"kivi k{bits}v{v_bits} d{d} R{R} {chunking}")


VALUE_BITS_DECODE = [
    # bits, v_bits, d, hg, dtype, R, T, rope, splits
    (4, 2, 128, 4, torch.bfloat16, 128, 700, 0.0, 0),      # matrix cores
    (4, 2, 64, 2, torch.bfloat16, 20, 300, 0.0, 3),
    (4, 2, 256, 8, torch.bfloat16, 40, 300, 0.0, 2),
    (4, 2, 128, 1, torch.bfloat16, 0, 161, 0.0, 1),
    (8, 4, 128, 4, torch.bfloat16, 16, 333, 0.0, 0),       # generic kernel
    (8, 2, 64, 2, torch.float32, 0, 257, 0.0, 5),
    (4, 2, 128, 4, torch.bfloat16, 128, 700, 500000.0, 0),  # rotary keys, generic
    (4, 2, 32, 1, torch.float32, 3, 98, 0.0, 0),
]


@pytest.mark.parametrize("bits,v_bits,d,hg,dtype,R,T,rope,splits", VALUE_BITS_DECODE)
def test_decode_kivi_value_bits(bits, v_bits, d, hg, dtype, R, T, rope, splits):
    w = small(synth.KIVI, bits, d, dtype, R, hg=hg, T=T, rope=rope, v_bits=v_bits)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q, ks, vs)
    want = oc.decode(0, H.values(q), rope_theta=rope)
    err = H.max_err(out, want)
    assert err <= H.ATOL, err


@pytest.mark.parametrize("chunking", ["one", "steps", "mixed"])
@pytest.mark.parametrize("bits,d,dtype", [(4, 32, torch.float32), (2, 128, torch.bfloat16),
                                          (8, 64, torch.bfloat16), (4, 256, torch.float32)])
def test_append_sym_bytes(bits, d, dtype, chunking):
    w = small(synth.SYM_TOKEN, bits, d, dtype, T=269)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=300)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"sym b{bits} d{d} {chunking}")


@pytest.mark.parametrize("chunking", ["one", "steps", "mixed"])
@pytest.mark.parametrize("d,shrink", [(128, 1.0), (64, 0.05), (32, 1.0), (256, 30.0)])
def test_append_fp8_bytes(d, shrink, chunking):
    """shrink < 1 makes the scales too small so large values saturate at 448;
    shrink > 1 pushes small values into the E4M3 subnormal range."""
    w = small(synth.FP8_E4M3, 8, d, T=269)
    k, v = synth.keys_values(w, device=DEV)
    ks, vs = synth.fp8_scales(k, v)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=300,
                                    scales=(ks * shrink, vs * shrink))
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"fp8 d{d} x{shrink} {chunking}")


@pytest.mark.parametrize("chunking", ["one", "steps", "mixed"])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float32),
                                     (32, torch.float32), (256, torch.bfloat16)])
def test_append_bf16_cache_bytes(d, dtype, chunking):
    """Unquantised baseline: bf16 input stored bit for bit, fp32 input rounded
    to nearest-even bfloat16."""
    w = small(synth.BF16_CACHE, 16, d, dtype, T=269)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=300)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"bf16 cache d{d} {chunking}")


@pytest.mark.parametrize("chunking", ["one", "steps", "mixed"])
@pytest.mark.parametrize("d,shrink", [(128, 1.0), (64, 0.02), (32, 1.0), (256, 3e3)])
def test_append_fp8_e5m2_bytes(d, shrink, chunking):
    """E5M2 pages; shrink < 1 saturates large values at 57344, shrink > 1
    pushes small values into the E5M2 subnormal range."""
    w = small(synth.FP8_E5M2, 8, d, T=269)
    k, v = synth.keys_values(w, device=DEV)
    ks, vs = synth.fp8_scales(k, v, 57344.0)
    cfg, cache, oc, *_ = run_append(w, CHUNKINGS[chunking](w.tokens), capacity=300,
                                    scales=(ks * shrink, vs * shrink))
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"e5m2 d{d} x{shrink} {chunking}")


def fp8_grid(e5):
    """Non-negative finite magnitudes of the FP8 format, from its definition:
    subnormals m * 2^(1 - bias - M), normals (1 + m / 2^M) * 2^(e - bias)."""
    M, bias, emax = (2, 15, 30) if e5 else (3, 7, 15)
    vals = [m * 2.0 ** (1 - bias - M) for m in range(2 ** M)]
    for e in range(1, emax + 1):
        for m in range(2 ** M):
            if not e5 and e == emax and m == 2 ** M - 1:
                continue                              # E4M3FN: S.1111.111 is NaN
            vals.append((1 + m / 2 ** M) * 2.0 ** (e - bias))
    return np.array(vals)


def rounding_edges(e5, scale):
    """Float32 inputs whose quotients by `scale` sit on or a few units around
    every FP8 number and every midpoint between neighbours, past the largest
    finite number, around the subnormal boundaries and at signed zeros."""
    g = fp8_grid(e5)
    mids = (g[:-1] + g[1:]) / 2
    top = g[-1]
    extra = [top * 1.0001, (top + (g[-1] - g[-2]) / 2), top * 1.5, top * 2, 1e30, 3e38,
             g[1] / 2, g[1] / 4, g[1] / 4 * 1.001, 1e-40, 1e-45]
    centres = np.float32(np.concatenate([g, mids, extra]) * scale)
    out = [centres]
    for k in (1, 2, 3, 4, 5, 8):
        up, down = centres.copy(), centres.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            down = np.nextafter(down, np.float32(0))
        out += [up, down]
    x = np.concatenate(out)
    return np.concatenate([x, -x, np.float32([0.0, -0.0])]).astype(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.3, 7.1e-3])
@pytest.mark.parametrize("scheme", [synth.FP8_E4M3, synth.FP8_E5M2])
def test_append_fp8_rounding_edges(scheme, scale):
    """Codes of values on and next to every FP8 rounding boundary (exact ties
    at scale 1; quotients a few units from a midpoint at the other scales,
    where the reciprocal product has to give way to the division) equal the
    oracle's nearest-even, saturating codes, in K rows and in V columns."""
    x = rounding_edges(scheme == synth.FP8_E5M2, scale)
    d = 128
    T = -(-x.size // d)
    flat = np.zeros(T * d, np.float32)
    flat[:x.size] = x
    w = small(scheme, 8, d, torch.float32, B=1, Hkv=1, hg=1, T=T)
    cfg = H.config(w, T)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, T)
    k = torch.from_numpy(flat.reshape(1, T, 1, d)).to(DEV)
    v = torch.from_numpy(np.roll(flat, 37).reshape(1, T, 1, d)).to(DEV)   # other positions
    ks = torch.full((1,), scale, dtype=torch.float32, device=DEV)
    H.append_chunks(cfg, cache, k, v, [5, T - 5], ks=ks, vs=ks, oc=oc)
    torch.cuda.synchronize()
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, f"fp8 edges scheme {scheme} scale {scale}")


def test_append_special_values():
    """Constant groups (s = 0), signed zeros and exact ties."""
    w = small(synth.KIVI, 2, 32, torch.float32, R=0, T=96)
    cfg = H.config(w, 96)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 96)
    k, v = synth.keys_values(w, device=DEV)
    k[:, 0:32, :, 3] = 2.5                                 # constant key channel in page 0
    k[:, 32:64, 1, :] = -0.0                               # whole page of -0 for head 1
    v[:, 5] = 0.0                                          # constant value row
    v[:, 6, :, :4] = torch.tensor([0.0, 0.5, 1.5, 3.0])    # exact ties at s = 1
    v[:, 6, :, 4:] = 1.0
    H.append_chunks(cfg, cache, k, v, [96], oc=oc)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "special values")


DECODE_CASES = [
    # scheme, bits, d, hg, dtype, R, T, rope, splits
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 700, 0.0, 0),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 161, 0.0, 1),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 100, 0.0, 0),     # ring only
    (synth.KIVI, 4, 128, 4, torch.bfloat16, 128, 700, 0.0, 3),
    (synth.KIVI, 8, 128, 8, torch.bfloat16, 16, 333, 0.0, 0),
    (synth.KIVI, 2, 64, 2, torch.float32, 0, 257, 0.0, 5),
    (synth.KIVI, 4, 32, 1, torch.float32, 3, 98, 0.0, 0),
    (synth.KIVI, 2, 256, 4, torch.bfloat16, 40, 300, 0.0, 2),
    (synth.KIVI, 2, 128, 4, torch.bfloat16, 128, 700, 500000.0, 0),
    (synth.KIVI, 4, 64, 2, torch.bfloat16, 20, 250, 10000.0, 4),
    (synth.SYM_TOKEN, 4, 32, 1, torch.float32, 0, 512, 0.0, 0),
    (synth.SYM_TOKEN, 2, 128, 4, torch.bfloat16, 0, 77, 0.0, 1),
    (synth.SYM_TOKEN, 8, 64, 8, torch.bfloat16, 0, 1, 0.0, 0),
    (synth.SYM_TOKEN, 4, 256, 2, torch.bfloat16, 0, 200, 500000.0, 3),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 333, 0.0, 0),
    (synth.FP8_E4M3, 8, 32, 1, torch.float32, 0, 65, 0.0, 2),
    (synth.FP8_E4M3, 8, 128, 4, torch.bfloat16, 0, 300, 500000.0, 0),
    (synth.FP8_E5M2, 8, 128, 4, torch.bfloat16, 0, 333, 0.0, 0),
    (synth.FP8_E5M2, 8, 64, 2, torch.bfloat16, 0, 97, 0.0, 3),
    (synth.FP8_E5M2, 8, 32, 1, torch.float32, 0, 65, 0.0, 2),
    (synth.FP8_E5M2, 8, 128, 8, torch.bfloat16, 0, 200, 500000.0, 0),
    (synth.BF16_CACHE, 16, 128, 4, torch.bfloat16, 0, 333, 0.0, 0),
    (synth.BF16_CACHE, 16, 32, 1, torch.float32, 0, 65, 0.0, 2),
    (synth.BF16_CACHE, 16, 64, 8, torch.bfloat16, 0, 1, 0.0, 0),
    (synth.BF16_CACHE, 16, 256, 2, torch.bfloat16, 0, 200, 500000.0, 3),
]


@pytest.mark.parametrize("scheme,bits,d,hg,dtype,R,T,rope,splits", DECODE_CASES)
def test_decode_parity(scheme, bits, d, hg, dtype, R, T, rope, splits):
    w = small(scheme, bits, d, dtype, R, hg=hg, T=T, rope=rope)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q, ks, vs)
    want = oc.decode(0, H.values(q), rope_theta=rope)
    err = H.max_err(out, want)
    assert err <= H.ATOL, err


MFMA_CASES = [
    # KIVI 2/4-bit pages on the matrix cores: every GQA width, head_dim 64/128/256
    (bits, d, hg, R, T, dtype)
    for bits in (2, 4)
    for (d, hg, R, T, dtype) in [(128, 1, 128, 300, torch.bfloat16), (128, 2, 0, 256, torch.float32),
                                 (128, 8, 128, 900, torch.bfloat16), (64, 4, 32, 500, torch.bfloat16),
                                 (256, 8, 64, 333, torch.bfloat16), (256, 1, 0, 96, torch.float32),
                                 (64, 8, 0, 64, torch.float32), (128, 4, 0, 32, torch.bfloat16)]
]


@pytest.mark.parametrize("bits,d,hg,R,T,dtype", MFMA_CASES)
def test_decode_mfma_pages(bits, d, hg, R, T, dtype):
    w = small(synth.KIVI, bits, d, dtype, R, hg=hg, T=T)
    cfg, cache, oc, *_ = run_append(w, [T], capacity=T + 40)
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q)
    err = H.max_err(out, oc.decode(0, H.values(q)))
    assert err <= H.ATOL, err


ROPE_CASES = [
    # KIVI 2-bit with keys cached before the rotary embedding, on the matrix
    # cores: GQA widths, head_dim 64/128, residual windows, ring-only caches,
    # split counts, a large base and a small one
    (d, hg, R, T, theta, splits)
    for (d, hg, R, T, theta, splits) in [
        (128, 4, 128, 700, 500000.0, 0), (128, 1, 0, 321, 10000.0, 0),
        (128, 2, 40, 1000, 500000.0, 5), (128, 8, 128, 260, 1e6, 1),
        (64, 4, 128, 90, 10000.0, 0), (64, 8, 16, 777, 500000.0, 3),
        (128, 4, 128, 3000, 500000.0, 64)]
]


@pytest.mark.parametrize("d,hg,R,T,theta,splits", ROPE_CASES)
def test_decode_rope_mfma(d, hg, R, T, theta, splits):
    w = small(synth.KIVI, 2, d, torch.bfloat16, R, hg=hg, T=T, rope=theta)
    cfg, cache, oc, *_ = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q)
    assert H.max_err(out, oc.decode(0, H.values(q), rope_theta=theta)) <= H.ATOL


FP8_CASES = [
    # FP8 pages on the matrix cores: GQA widths, head_dim 64/128/256, partial
    # last pages (T % 32 = 0, 1, 17, 31), single-page caches, split counts
    (d, hg, T, dtype, splits)
    for (d, hg, T, dtype, splits) in [
        (128, 4, 333, torch.bfloat16, 0), (128, 1, 32, torch.bfloat16, 0),
        (128, 2, 257, torch.float32, 3), (128, 8, 95, torch.bfloat16, 1),
        (64, 4, 1, torch.bfloat16, 0), (64, 8, 500, torch.float32, 7),
        (256, 4, 161, torch.bfloat16, 2), (256, 1, 5, torch.float32, 0),
        (128, 4, 1024, torch.bfloat16, 40)]
]


@pytest.mark.parametrize("d,hg,T,dtype,splits", FP8_CASES)
def test_decode_fp8_mfma(d, hg, T, dtype, splits):
    w = small(synth.FP8_E4M3, 8, d, dtype, 0, hg=hg, T=T)
    cfg, cache, oc, k, v, ks, vs = run_append(w, [T], capacity=T + 40)
    cfg.num_splits = splits
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, T, q, ks, vs)
    assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL


def test_decode_fp8_unwritten_bytes_are_ignored():
    """The cache beyond the last token holds 0xFF bytes (an E4M3 NaN pattern):
    the partial last page must not let them into the scores or the output."""
    w = small(synth.FP8_E4M3, 8, 128, torch.bfloat16, 0, hg=4, T=45)
    cfg = H.config(w, 96)
    cache = kvq.alloc_cache(cfg, zero=False)
    cache.fill_(0xFF)
    oc = H.oracle_cache(w, 96)
    k, v = synth.keys_values(w, device=DEV)
    ks, vs = synth.fp8_scales(k, v)
    H.append_chunks(cfg, cache, k, v, [45], ks=ks, vs=vs, oc=oc)
    q = synth.query(w, device=DEV)
    out = H.decode(cfg, cache, 0, 45, q, ks, vs)
    assert torch.isfinite(out).all()
    assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL


@pytest.mark.parametrize("bits,v_bits,dtype", [
    (2, 0, torch.float32), (4, 0, torch.float32),       # generic (vector-ALU) kernel
    (2, 0, torch.bfloat16), (4, 0, torch.bfloat16),     # matrix-core kernel
    (4, 2, torch.bfloat16)])
def test_decode_mfma_dynamic_range(bits, v_bits, dtype):
    """Keys and values over many orders of magnitude: per-channel scales from
    1e-4 to 1e3, so q * s spans far more than fp16's 11 bits and the hi/lo
    split carries the accuracy; value rows from 1e-2 to 1e2; peaked attention
    through large queries. The plain max-abs 2e-3 bound, at every output
    magnitude. bf16 inputs run on the matrix-core kernel (f16 hi/lo key
    operand, bf16 hi/lo weights), f32 inputs on the generic kernel."""
    w = small(synth.KIVI, bits, 128, dtype, 32, hg=4, T=600, v_bits=v_bits)
    k, v = synth.keys_values(w, device=DEV)
    ch = torch.logspace(-4, 3, 128, device=DEV)
    k = (k.float() * ch.view(1, 1, 1, 128)).to(dtype).contiguous()
    v = (v.float() * torch.logspace(-2, 2, 600, device=DEV).view(1, 600, 1, 1)).to(dtype).contiguous()
    cfg = H.config(w, 640)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 640)
    H.append_chunks(cfg, cache, k, v, [600], oc=oc)
    q = (synth.query(w, device=DEV).float() * 3.0).to(dtype).contiguous()
    out = H.decode(cfg, cache, 0, 600, q)
    want = oc.decode(0, H.values(q))
    err = H.max_err(out, want)
    print(f"[dynamic range] b{bits} v{v_bits or bits} {dtype}: max|out| "
          f"{float(np.max(np.abs(want))):.1f}, max-abs error {err:.2e}", flush=True)
    assert err <= H.ATOL


def _one_page_keys(w, kvals):
    """[B, 32, Hkv, d] keys, zero except the listed (token, channel) -> value
    entries (the same in every sequence and KV head)."""
    k = torch.zeros(w.batch, 32, w.kv_heads, w.head_dim, dtype=torch.float32)
    for (t, c), x in kvals.items():
        k[:, t, :, c] = x
    return k.to(w.in_dtype).to(DEV).contiguous()


@pytest.mark.parametrize("bits,v_bits", [(2, 0), (4, 0), (4, 2)])
def test_decode_f16_range_guard_kivi(bits, v_bits):
    """A key channel whose scaled query q * s * sm_scale * log2(e) exceeds the
    f16 maximum (65504) on the matrix-core kernel. One page, keys built so the
    quantisation is exact (per-channel minimum 0): channel 0 gives token X
    code L and token Y code L-1 or so, channel 1 gives Y the top code. With the
    true q', X wins by thousands of log2 units; had q' saturated at the f16
    maximum, Y would win by hundreds. Values: X's row all +1, Y's all -1,
    others 0 -- so the output is +1 exactly, and -1 if the range were lost."""
    w = small(synth.KIVI, bits, 128, torch.bfloat16, 0, B=1, Hkv=1, hg=4, T=32, v_bits=v_bits)
    L = float((1 << bits) - 1)
    X, Y = 3, 17
    # channel 0: X = L * 2^17, Y = (L - 1) * 2^17, others 0 -> s0 = 2^17, codes L, L - 1
    # channel 1: Y = 2^20 (code L), others 0 -> s1 = fl(2^20 / L)
    k = _one_page_keys(w, {(X, 0): L * 2.0 ** 17, (Y, 0): (L - 1) * 2.0 ** 17, (Y, 1): 2.0 ** 20})
    v = torch.zeros(1, 32, 1, 128, dtype=torch.float32)
    v[0, X], v[0, Y] = 1.0, -1.0
    v = v.to(torch.bfloat16).to(DEV).contiguous()
    # q' = q * s * qs, qs = log2(e) / sqrt(128); score(X) - score(Y) = q0' - L q1'
    qs = float(np.log2(np.e) / np.sqrt(128.0))
    s0, s1 = 2.0 ** 17, float(np.float32(2.0 ** 20) / np.float32(L))
    q0 = 8.0                                  # q0' = 8 * 2^17 * qs ~ 1.34e5 > 65504
    q1 = None
    for cand in np.arange(4.0, 0.0, -2.0 ** -7):  # bf16-exact candidates, largest first
        q1p = cand * s1 * qs
        sat = 2 * 65504.0                      # hi + lo of a saturated f16 split
        if q1p < 65504 and q0 * s0 * qs - L * q1p > 500 and sat - L * q1p < -200:
            q1 = float(cand)
            break
    assert q1 is not None
    q = torch.zeros(1, 4, 128, dtype=torch.float32)
    q[0, :, 0], q[0, :, 1] = q0, q1
    q = q.to(torch.bfloat16).to(DEV).contiguous()
    cfg = H.config(w, 32)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 32)
    H.append_chunks(cfg, cache, k, v, [32], oc=oc)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "range-guard page")
    out = H.decode(cfg, cache, 0, 32, q)
    ref = oc.decode(0, H.values(q))
    assert np.allclose(ref, 1.0, atol=1e-6)    # the construction: X takes all the weight
    assert H.max_err(out, ref) <= H.ATOL


def test_decode_f16_range_guard_fp8():
    """FP8 E4M3 keys with a per-head scale so large that q * k_scale *
    sm_scale * log2(e) exceeds the f16 maximum: token X (channel 0 at 448)
    must win over Y (channel 0 at 320, channel 1 at 448); with q' saturated at
    the f16 maximum Y would win. Values: X's row +1, Y's -1."""
    w = small(synth.FP8_E4M3, 8, 128, torch.bfloat16, 0, B=1, Hkv=1, hg=4, T=32)
    ksc = 2.0 ** 20
    X, Y = 5, 22
    k = _one_page_keys(w, {(X, 0): 448 * ksc, (Y, 0): 320 * ksc, (Y, 1): 448 * ksc})
    v = torch.zeros(1, 32, 1, 128, dtype=torch.float32)
    v[0, X], v[0, Y] = 1.0, -1.0
    v = v.to(torch.bfloat16).to(DEV).contiguous()
    qs = float(np.log2(np.e) / np.sqrt(128.0))
    q0p = 1.0 * ksc * qs                       # ~1.34e5 > 65504
    sat = 2 * 65504.0
    q1 = None
    for cand in np.arange(1.0, 0.0, -2.0 ** -9):
        q1p = cand * ksc * qs
        if q1p < 65504 and 128 * q0p - 448 * q1p > 1e4 and 128 * sat - 448 * q1p < -1e4:
            q1 = float(cand)
            break
    assert q1 is not None
    q = torch.zeros(1, 4, 128, dtype=torch.float32)
    q[0, :, 0], q[0, :, 1] = 1.0, q1
    q = q.to(torch.bfloat16).to(DEV).contiguous()
    ks = torch.full((1,), ksc, dtype=torch.float32, device=DEV)
    vs = torch.ones(1, dtype=torch.float32, device=DEV)
    cfg = H.config(w, 32)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 32)
    H.append_chunks(cfg, cache, k, v, [32], ks=ks, vs=vs, oc=oc)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "fp8 range-guard page")
    out = H.decode(cfg, cache, 0, 32, q, ks, vs)
    ref = oc.decode(0, H.values(q))
    assert np.allclose(ref, 1.0, atol=1e-6)
    assert H.max_err(out, ref) <= H.ATOL


def test_decode_split_invariance_and_determinism():
    w = small(synth.KIVI, 2, 128, torch.bfloat16, 128, hg=4, T=1500)
    cfg, cache, oc, *_ = run_append(w, [w.tokens], capacity=1600)
    q = synth.query(w, device=DEV)
    want = oc.decode(0, H.values(q))
    outs = []
    for s in (1, 2, 7, 0, 64):
        cfg.num_splits = s
        o1 = H.decode(cfg, cache, 0, w.tokens, q)
        o2 = H.decode(cfg, cache, 0, w.tokens, q)
        assert torch.equal(o1, o2), s                       # run twice: identical
        assert H.max_err(o1, want) <= H.ATOL, s
        outs.append(o1)
    for o in outs[1:]:
        assert float((o - outs[0]).abs().max()) < 1e-4


def test_shared_workspace_across_kernels():
    """One workspace serves, one call after another, the matrix-core KIVI
    kernel, the generic kernel and the FP8 kernel at several split counts and
    query counts: each result stays within 2e-3 of the oracle, and after every
    call the whole workspace (arrival counters and split partials) is zero
    again, so no call reads partials another call left behind."""
    cases = []
    for scheme, bits, splits in ((synth.KIVI, 2, 7), (synth.KIVI, 8, 5), (synth.FP8_E4M3, 8, 3),
                                 (synth.KIVI, 2, 2), (synth.KIVI, 4, 0)):
        w = small(scheme, bits, 128, torch.bfloat16, 0 if scheme == synth.FP8_E4M3 else 32, B=3, hg=4, T=700)
        cfg, cache, oc, k, v, ks, vs = run_append(w, [w.tokens], capacity=740)
        cfg.num_splits = splits
        cases.append((w, cfg, cache, oc, ks, vs, splits))
    nq = 3
    need = max(nq * kvq.kvq_cache_bytes(c[1], c[0].tokens, kvq.KVQ_BYTES_WORKSPACE) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for rnd in range(2):
        for w, cfg, cache, oc, ks, vs, splits in cases:
            q = synth.query(w, device=DEV, tag=rnd)
            out = H.decode(cfg, cache, 0, w.tokens, q, ks, vs, ws=ws)
            assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL, (w.name, splits)
            assert int(ws.count_nonzero()) == 0, (w.name, splits)
            qm = torch.stack([synth.query(w, device=DEV, tag=10 + i) for i in range(nq)], dim=1).contiguous()
            om = torch.empty(qm.shape, dtype=torch.float32, device=DEV)
            kvq.kvq_decode_attention_multi(cfg, cache, 0, w.tokens, qm, om, ws, k_scale=ks, v_scale=vs)
            assert H.max_err(om, oc.decode_multi(0, H.values(qm))) <= H.ATOL, (w.name, splits, nq)
            assert int(ws.count_nonzero()) == 0, (w.name, splits, nq)


def test_append_determinism_and_noop():
    w = small(synth.KIVI, 4, 128, torch.bfloat16, 128, T=500)
    cfg, c1, *_ = run_append(w, [w.tokens], capacity=512)
    cfg, c2, *_ = run_append(w, [w.tokens], capacity=512)
    assert torch.equal(c1, c2)
    k, v = synth.keys_values(w, device=DEV)
    before = c1.clone()
    kvq.kvq_quantize_append(cfg, c1, 0, w.tokens, 0, k, v)    # new_tokens = 0
    torch.cuda.synchronize()
    assert torch.equal(before, c1)


def test_decode_after_incremental_appends():
    """Decode interleaved with one-token appends, crossing page flushes."""
    w = small(synth.KIVI, 2, 128, torch.bfloat16, 16, hg=4, T=120)
    cfg = H.config(w, 128)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 128)
    k, v = synth.keys_values(w, device=DEV)
    q = synth.query(w, device=DEV)
    ws = kvq.alloc_workspace(cfg)
    H.append_chunks(cfg, cache, k, v, [40], oc=oc)
    for t in range(40, w.tokens):
        kvq.kvq_quantize_append(cfg, cache, 0, t, 1, k[:, t:t + 1].contiguous(),
                                v[:, t:t + 1].contiguous())
        oc.append(0, H.host(k[:, t:t + 1]), H.host(v[:, t:t + 1]))
        if t % 9 == 0 or t == w.tokens - 1:
            out = H.decode(cfg, cache, 0, t + 1, q, ws=ws)
            assert H.max_err(out, oc.decode(0, H.values(q))) <= H.ATOL, t
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "incremental")


def test_multi_layer_addressing():
    w = small(synth.KIVI, 2, 64, torch.bfloat16, 32, hg=2, T=200)
    cfg = H.config(w, 200, layers=3)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, 200, layers=3)
    for layer in (2, 0):
        k, v = synth.keys_values(w, layer=layer, device=DEV)
        H.append_chunks(cfg, cache, k, v, [200], layer=layer, oc=oc)
    want, mask = oc.cache_image()
    H.compare_bytes(cache.cpu().numpy(), want, mask, "layers")
    q = synth.query(w, device=DEV)
    for layer in (0, 2):
        out = H.decode(cfg, cache, layer, 200, q)
        assert H.max_err(out, oc.decode(layer, H.values(q))) <= H.ATOL


SCORE_RAMPS = [
    # bits, d, hg, R, T, ramp: keys scaled by 1 + ramp * t / T, so the running
    # maximum of the scores grows page after page, by less than and by more than
    # the kernels' rescaling slack (8 in log2 units)
    (2, 128, 4, 128, 1400, 3.0), (2, 128, 4, 128, 1400, 12.0), (2, 64, 1, 0, 700, 25.0),
    (4, 128, 4, 128, 1400, 12.0), (4, 128, 8, 32, 900, 6.0), (2, 128, 2, 128, 900, -0.9),
]


@pytest.mark.parametrize("bits,d,hg,R,T,ramp", SCORE_RAMPS)
def test_decode_growing_scores(bits, d, hg, R, T, ramp):
    """Decode where later tokens score ever higher (or, for a negative ramp,
    lower): the online softmax must rescale correctly however far the maximum
    moves between pages."""
    w = small(synth.KIVI, bits, d, torch.bfloat16, R, hg=hg, T=T)
    cfg = H.config(w, T + 40)
    cache = kvq.alloc_cache(cfg)
    oc = H.oracle_cache(w, T + 40)
    k, v = synth.keys_values(w, device=DEV)
    q = synth.query(w, device=DEV)
    # keys along the first query head's direction, growing with t
    t = torch.arange(T, device=DEV, dtype=torch.float32)
    scale = (1.0 + ramp * t / T).view(1, T, 1, 1)
    qdir = q.float()[:, ::hg].unsqueeze(1)                      # [B, 1, Hkv, d]
    k = (k.float() * 0.3 + 2.0 * qdir * scale).to(torch.bfloat16)
    H.append_chunks(cfg, cache, k, v, [T], oc=oc)
    torch.cuda.synchronize()
    out = H.decode(cfg, cache, 0, T, q)
    err = H.max_err(out, oc.decode(0, H.values(q)))
    assert err <= H.ATOL, err
