"""Seeded synthetic inputs for the five workloads (shapes and distributions only).

This module holds none of the quantisation or attention arithmetic; the HIP
library and the oracle both receive the tensors it makes. Distributions:

* keys ~ N(0,1) with a few outlier channels multiplied by a factor, the
  channels drawn once per (layer, KV head) and shared by every sequence and
  token ("Quantizing the KV cache": keys have a few channels large in every
  token; KIVI: persistent outlier channels);
* values ~ N(0,1) with floor(frac * T) outlier tokens per sequence multiplied
  by a factor, shared by the sequence's KV heads (KIVI: values have sporadic
  outlier tokens);
* optionally, isolated elements of keys and values multiplied by a factor
  (sparse outliers inside otherwise ordinary vectors, the case KVQuant's
  dense-and-sparse pages address);
* queries ~ N(0,1).
Factors are applied in float32 before rounding to bfloat16 (round to nearest
even). Every tensor comes from its own torch generator seeded by (workload,
layer, tensor), on the requested device.
"""

from dataclasses import dataclass, replace

import torch

KIVI, SYM_TOKEN, FP8_E4M3, BF16_CACHE, FP8_E5M2, FP8K_SYMV, FP8K_KIVIV = 0, 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    scheme: int
    bits: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    tokens: int
    residual: int = 0
    in_dtype: torch.dtype = torch.bfloat16
    q_dtype: torch.dtype = torch.bfloat16
    k_outlier_channels: int = 0
    k_outlier_factor: float = 1.0
    v_outlier_frac: float = 0.0
    v_outlier_factor: float = 1.0
    rope_theta: float = 0.0
    layers: int = 1
    v_bits: int = 0          # KIVI value-code bits; 0 = the key bits
    outliers: int = 0        # KIVI: 1 = dense-and-sparse pages (a config field, no data)
    spike_frac: float = 0.0  # fraction of single key and value elements scaled by spike_factor
    spike_factor: float = 1.0


WORKLOADS = {
    # 1 layer, 1 sequence, 4 KV heads x 32, 512 tokens, fp32, 2 key channels x10,
    # symmetric per-head-per-token 4-bit; one fp32 query per head
    "tiny": Workload("tiny", 0, SYM_TOKEN, 4, 1, 4, 4, 32, 512, in_dtype=torch.float32,
                     q_dtype=torch.float32, k_outlier_channels=2, k_outlier_factor=10.0),
    # KIVI 2-bit, Llama-3-8B layer shape, batch 16, context 4096, R = 128
    "kivi2": Workload("kivi2", 1, KIVI, 2, 16, 32, 8, 128, 4096, residual=128,
                      k_outlier_channels=4, k_outlier_factor=20.0,
                      v_outlier_frac=0.01, v_outlier_factor=10.0),
    # FP8 E4M3 per-head scale, batch 64, context 8192 (+1 appended token)
    "fp8": Workload("fp8", 2, FP8_E4M3, 8, 64, 32, 8, 128, 8192,
                    k_outlier_channels=4, k_outlier_factor=20.0),
    # INT4 KIVI, batch 32, context 32768, R = 128
    "int4": Workload("int4", 3, KIVI, 4, 32, 32, 8, 128, 32768, residual=128,
                     k_outlier_channels=4, k_outlier_factor=20.0,
                     v_outlier_frac=0.01, v_outlier_factor=10.0),
    # KIVI with 4-bit keys and 2-bit values at the kivi2 shape (keys kept wider:
    # their outlier channels make rounding cost them more than values)
    "kivi_k4v2": Workload("kivi_k4v2", 5, KIVI, 4, 16, 32, 8, 128, 4096, residual=128,
                          k_outlier_channels=4, k_outlier_factor=20.0,
                          v_outlier_frac=0.01, v_outlier_factor=10.0, v_bits=2),
    # long context 2-bit, batch 1, 1,048,576 tokens, keys pre-RoPE (theta 500000)
    "longctx": Workload("longctx", 4, KIVI, 2, 1, 32, 8, 128, 1 << 20, residual=128,
                        k_outlier_channels=4, k_outlier_factor=20.0,
                        v_outlier_frac=0.01, v_outlier_factor=10.0, rope_theta=500000.0),
}


def scaled(w, **kw):
    """A copy of workload `w` with some fields replaced (smaller test sizes)."""
    return replace(w, **kw)


def _gen(w, layer, tensor_id, device):
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * w.wid + 7_919 * layer + tensor_id)
    return g


def outlier_channels(w, layer, device="cpu"):
    """[kv_heads, n] sorted channel indices per KV head."""
    g = _gen(w, layer, 11, "cpu")
    rows = [torch.randperm(w.head_dim, generator=g)[: w.k_outlier_channels].sort().values
            for _ in range(w.kv_heads)]
    return torch.stack(rows).to(device) if rows and w.k_outlier_channels else None


def outlier_tokens(w, layer, tokens, device="cpu"):
    """[batch, n] token positions per sequence, n = floor(frac * tokens)."""
    n = int(w.v_outlier_frac * tokens)
    if n == 0:
        return None
    g = _gen(w, layer, 12, "cpu")
    rows = [torch.randperm(tokens, generator=g)[:n].sort().values for _ in range(w.batch)]
    return torch.stack(rows).to(device)


def keys_values(w, layer=0, tokens=None, device="cpu", token_offset=0, tag=0):
    """(K, V) of shape [batch, tokens, kv_heads, head_dim] in w.in_dtype.

    `tag` selects an independent draw (e.g. the tokens appended by decode steps);
    outlier channels stay those of (w, layer)."""
    T = w.tokens if tokens is None else tokens
    shape = (w.batch, T, w.kv_heads, w.head_dim)
    k = torch.randn(shape, generator=_gen(w, layer, 1 + 100 * tag, device), device=device,
                    dtype=torch.float32)
    v = torch.randn(shape, generator=_gen(w, layer, 2 + 100 * tag, device), device=device,
                    dtype=torch.float32)
    ch = outlier_channels(w, layer, device)
    if ch is not None:
        f = torch.ones(w.kv_heads, w.head_dim, device=device)
        f.scatter_(1, ch, w.k_outlier_factor)
        k.mul_(f.view(1, 1, w.kv_heads, w.head_dim))
    if w.spike_frac > 0:
        # isolated large elements (sparse outliers), drawn independently for K and V
        for x, tid in ((k, 4), (v, 5)):
            u = torch.rand(shape, generator=_gen(w, layer, tid + 100 * tag, device), device=device)
            x.mul_(torch.where(u < w.spike_frac, w.spike_factor, 1.0))
    if tag == 0 and token_offset == 0:
        pos = outlier_tokens(w, layer, T, device)
        if pos is not None:
            f = torch.ones(w.batch, T, device=device)
            f.scatter_(1, pos, w.v_outlier_factor)
            v.mul_(f.view(w.batch, T, 1, 1))
    return k.to(w.in_dtype), v.to(w.in_dtype)


def query(w, layer=0, device="cpu", tag=0):
    """[batch, q_heads, head_dim] in w.q_dtype."""
    q = torch.randn((w.batch, w.q_heads, w.head_dim), generator=_gen(w, layer, 3 + 100 * tag,
                                                                      device),
                    device=device, dtype=torch.float32)
    return q.to(w.q_dtype)


def fp8_scales(k, v, fmax=448.0):
    """Static per-KV-head scales: max |x| over the head's context / fmax, the
    format's largest finite value (448 for E4M3, 57344 for E5M2; the caller's
    calibration of the FP8 range), float32 [kv_heads] each."""
    ks = k.float().abs().amax(dim=(0, 1, 3)) / fmax
    vs = v.float().abs().amax(dim=(0, 1, 3)) / fmax
    return ks.contiguous(), vs.contiguous()
