"""Shared helpers of the GPU parity tests: run the HIP library and the oracle on
the same seeded inputs and compare.

Inputs come from ``synth`` (seeded torch generators); the oracle gets host
copies of exactly the tensors the library gets. Nothing here computes any part
of the method itself: encodings and attention come from ``oracle``.
"""

import numpy as np
import torch

import kv_cache_quantisation_amd as kvq
import synth
from oracle import accounting, attention, codec, rope
from oracle.cache import OracleCache, bf16_bits_to_f32

ATOL = 2e-3  # max-abs tolerance of decode outputs against the fp64 oracle

DT = {torch.bfloat16: kvq.KVQ_BF16, torch.float32: kvq.KVQ_F32}


def host(x):
    """Host copy of an input in the oracle's convention: bf16 -> uint16 bit
    patterns, f32 -> float32."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy().astype(np.float32, copy=False)


def values(x):
    """Exact float32 values of a bf16/f32 tensor (host)."""
    h = host(x)
    return bf16_bits_to_f32(h) if h.dtype == np.uint16 else h


def config(w, capacity=None, num_splits=0, layers=None):
    return kvq.make_config(w.scheme, w.bits, layers or w.layers, w.q_heads, w.kv_heads,
                           w.head_dim, w.batch, capacity or w.tokens, residual=w.residual,
                           in_dtype=DT[w.in_dtype], q_dtype=DT[w.q_dtype],
                           rope_theta=w.rope_theta, num_splits=num_splits, v_bits=w.v_bits,
                           outliers=w.outliers)


def oracle_cache(w, capacity=None, layers=None):
    return OracleCache(w.scheme, w.bits, layers or w.layers, w.batch, w.kv_heads, w.head_dim,
                       capacity or w.tokens, residual=w.residual,
                       in_dtype="bf16" if w.in_dtype == torch.bfloat16 else "f32",
                       v_bits=w.v_bits or None, outliers=w.outliers)


def append_chunks(cfg, cache, k, v, chunks, layer=0, ks=None, vs=None, oc=None):
    """Appends k/v [B, T, H, d] (device) in the given chunk lengths through the
    library and, if `oc` is given, the oracle."""
    t = 0
    for n in chunks:
        kc = k[:, t:t + n].contiguous()
        vc = v[:, t:t + n].contiguous()
        kvq.kvq_quantize_append(cfg, cache, layer, t, n, kc, vc, ks, vs)
        if oc is not None:
            oc.append(layer, host(kc), host(vc),
                      None if ks is None else host(ks), None if vs is None else host(vs))
        t += n
    return t


def compare_bytes(gpu_bytes, want, mask, what=""):
    """Bit-exact comparison of the defined bits; reports the first mismatch."""
    got = np.asarray(gpu_bytes, np.uint8)
    assert got.size == want.size, (what, got.size, want.size)
    bad = np.nonzero((got ^ want) & mask)[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} bytes differ; first at {i}: "
                             f"gpu {got[i]:#04x} oracle {want[i]:#04x} mask {mask[i]:#04x}")


def decode(cfg, cache, layer, tokens, q, ks=None, vs=None, ws=None):
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = kvq.alloc_workspace(cfg, tokens, device=q.device)
    kvq.kvq_decode_attention(cfg, cache, layer, tokens, q, out, ws, k_scale=ks, v_scale=vs)
    return out


def max_err(gpu_out, want):
    return float(np.max(np.abs(gpu_out.detach().cpu().numpy().astype(np.float64) - want)))


# ---- per-(sequence, KV head) oracle pieces for large workloads ---------------

def oracle_dequant_head(w, kf, vf, T, ks=None, vs=None):
    """Dequantised keys/values [T, d] (float64) of one (sequence, KV head) of a
    cache holding T tokens, from its exact input values kf, vf [T, d]."""
    d = w.head_dim
    if w.scheme == synth.KIVI:
        q, _ = accounting.flush_plan(T, w.residual)
        kh = np.array(kf[:T], np.float64)
        vh = np.array(vf[:T], np.float64)
        if q:
            kg = kf[:q].reshape(q // 32, 32, d)
            vg = vf[:q].reshape(q // 32, 32, d)
            c, s, z = codec.kivi_quantize(kg, w.bits, axis=1)
            kh[:q] = codec.kivi_dequantize(c, s, z, axis=1).reshape(q, d)
            c, s, z = codec.kivi_quantize(vg, w.v_bits or w.bits, axis=2)
            vh[:q] = codec.kivi_dequantize(c, s, z, axis=2).reshape(q, d)
        return kh, vh
    if w.scheme == synth.BF16_CACHE:
        return codec.bf16_decode(codec.bf16_encode(kf[:T])), codec.bf16_decode(codec.bf16_encode(vf[:T]))
    if w.scheme == synth.SYM_TOKEN:
        c, s = codec.sym_quantize(kf[:T], w.bits, axis=1)
        kh = codec.sym_dequantize(c, s, axis=1)
        c, s = codec.sym_quantize(vf[:T], w.bits, axis=1)
        return kh, codec.sym_dequantize(c, s, axis=1)
    f = "e5m2" if w.scheme == synth.FP8_E5M2 else "e4m3"
    kh = codec.fp8_dequantize(codec.fp8_quantize(kf[:T], ks, f), ks, f)
    vh = codec.fp8_dequantize(codec.fp8_quantize(vf[:T], vs, f), vs, f)
    return kh, vh


def oracle_attend_head(w, q_rows, kh, vh, T):
    """fp64 attention of the query rows of one KV head's GQA group."""
    sm = 1.0 / np.sqrt(w.head_dim)
    q_rows = np.asarray(q_rows, np.float64)
    if w.rope_theta > 0:
        kh = rope.rotate(kh, np.arange(T), w.rope_theta)
        q_rows = rope.rotate(q_rows, np.full(len(q_rows), T - 1), w.rope_theta)
    return np.stack([attention.attend(qr, kh, vh, sm) for qr in q_rows])
