"""Benchmark of the quantised-KV-cache hot path on one MI355X.

A step is one decode step of a 32-layer model of Llama-3-8B layer shape
(32 query / 8 KV heads, head_dim 128) at batch 16 over a KIVI 2-bit cache with
a 128-token bf16 residual window: for every layer, quantize-append of the new
token of each sequence (flushing a 32-token group whenever the window fills),
then decode attention of one query per sequence over all cached tokens. The
32 layers have distinct caches (about 2 GB, far beyond the 256 MB Infinity
Cache), so every decode reads its cache from HBM. The context starts at 4096
tokens (the workload's size) and grows by one token per step.

value = algorithmic bytes of the K timed steps / their wall time (GB/s):
decode reads the packed codes, fp32 scales/offsets, the residual ring, the
query and writes the output; append reads the new K/V rows and writes the ring
(and, on flush steps, reads 32 ring rows and writes the page).

Also reported: quantize-append tokens/s for the 4096-token prefill of each
layer, the decode kernel against the HBM roofline (per-launch HIP events on
the launch stream), and the CPU oracle on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kv_cache_quantisation_amd as kvq  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
METRIC = "decode-attn effective HBM GB/s (% of MI355X peak) + quantize-append tokens/s"


def kivi_q(T, R):
    return 32 * (max(0, T - R) // 32)


def decode_bytes(w, T, in_bytes=2, q_bytes=2):
    """Algorithmic bytes of one decode call over T tokens (all sequences/heads)."""
    page = 2 * 32 * w.head_dim * w.bits // 8 + 8 * w.head_dim + 256
    q = kivi_q(T, w.residual)
    per_unit = (q // 32) * page + (T - q) * 2 * w.head_dim * in_bytes
    hg = w.q_heads // w.kv_heads
    per_unit += hg * w.head_dim * (q_bytes + 4)
    return w.batch * w.kv_heads * per_unit


def append_bytes(w, T_old, n, in_bytes=2):
    """Algorithmic bytes of appending n tokens to a T_old-token KIVI cache."""
    d, R = w.head_dim, w.residual
    page = 2 * 32 * d * w.bits // 8 + 8 * d + 256
    q0, q1 = kivi_q(T_old, R), kivi_q(T_old + n, R)
    row = 2 * d * in_bytes                         # one K row + one V row
    rd = n * row                                   # new tokens
    from_ring = max(0, min(q1, T_old) - q0)        # flushed tokens that sat in the ring
    rd += from_ring * row
    wr = ((q1 - q0) // 32) * page + max(0, T_old + n - max(q1, T_old)) * row
    return w.batch * w.kv_heads * (rd + wr)


def gpu_bench(args, w):
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L, W, K = args.layers, args.warmup, args.steps
    T0 = w.tokens
    cap = T0 + W + K + 64
    cfg = kvq.make_config(w.scheme, w.bits, L, w.q_heads, w.kv_heads, w.head_dim, w.batch, cap,
                          residual=w.residual)
    cache = kvq.alloc_cache(cfg, device=dev, zero=False)
    ws = kvq.alloc_workspace(cfg, device=dev)
    stream = torch.cuda.current_stream()

    # prefill every layer's 4096-token context (timed per layer: quantize-append)
    pre_ms = []
    for layer in range(L):
        k, v = synth.keys_values(w, layer=layer, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_quantize_append(cfg, cache, layer, 0, T0, k, v, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        pre_ms.append(e0.elapsed_time(e1))
        del k, v
    prefill_ms = sorted(pre_ms)[len(pre_ms) // 2]
    append_tps = w.batch * T0 / (prefill_ms * 1e-3)
    prefill_bytes = append_bytes(w, 0, T0)

    # per-layer inputs of the decode steps
    news = [synth.keys_values(w, layer=layer, tokens=W + K, device=dev, tag=1) for layer in range(L)]
    qs = [synth.query(w, layer=layer, device=dev) for layer in range(L)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device=dev) for q in qs]

    # one contiguous [B, 1, H, d] tensor per (layer, step), made before timing
    news = [(kn.unbind(1), vn.unbind(1)) for kn, vn in news]
    news = [([x.unsqueeze(1).contiguous() for x in kl], [x.unsqueeze(1).contiguous() for x in vl])
            for kl, vl in news]

    def step(i):
        T = T0 + i
        for layer in range(L):
            kvq.kvq_quantize_append(cfg, cache, layer, T, 1, news[layer][0][i], news[layer][1][i],
                                    stream=stream)
            kvq.kvq_decode_attention(cfg, cache, layer, T + 1, qs[layer], outs[layer], ws,
                                     stream=stream)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(W, W + K):
        step(i)
    s1.record(stream)
    torch.cuda.synchronize()
    total_ms = s0.elapsed_time(s1)
    total_bytes = sum(L * (append_bytes(w, T0 + i, 1) + decode_bytes(w, T0 + i + 1))
                      for i in range(W, W + K))
    gbs = total_bytes / (total_ms * 1e-3) / 1e9

    # decode kernel alone: per-launch event pairs on the launch stream
    T_end = T0 + W + K
    n_rep = 3
    evs = []
    for _ in range(n_rep):
        for layer in range(L):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            kvq.kvq_decode_attention(cfg, cache, layer, T_end, qs[layer], outs[layer], ws,
                                     stream=stream)
            b.record(stream)
            evs.append((a, b))
    torch.cuda.synchronize()
    launch_us = [a.elapsed_time(b) * 1e3 for a, b in evs]
    avg_us = sum(launch_us) / len(launch_us)
    per_launch = decode_bytes(w, T_end)
    achieved = per_launch / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "kvq decode (split + merge)", "avg_launch_us": round(avg_us, 2),
                "bytes_per_launch": per_launch}
    return {
        "ms_per_step": total_ms / K, "gbs": gbs, "append_tps": append_tps,
        "prefill_ms_per_layer": prefill_ms, "prefill_gbs": prefill_bytes / (prefill_ms * 1e-3) / 1e9,
        "roofline": roofline, "cache_bytes": int(cache.numel()),
    }


def cpu_baseline(w, budget_s=12.0, max_units=256):
    """The oracle (as it stands) on a bounded sample: decode attention of whole
    (sequence, KV head) units of one layer at the workload's context, each unit
    quantised, dequantised and attended by the oracle on the host."""
    import numpy as np
    from oracle.cache import OracleCache
    from threadpoolctl import threadpool_limits
    k, v = synth.keys_values(w, layer=0, device="cpu")
    q = synth.query(w, layer=0, device="cpu")
    raw_k = k.view(torch.int16).numpy().view(np.uint16)
    raw_v = v.view(torch.int16).numpy().view(np.uint16)
    hg = w.q_heads // w.kv_heads
    T = w.tokens
    one = synth.scaled(w, batch=1, kv_heads=1, q_heads=hg)
    done, t0 = 0, time.perf_counter()
    units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    with threadpool_limits(limits=1):
        for b, h in units[:max_units]:
            oc = OracleCache(w.scheme, w.bits, 1, 1, 1, w.head_dim, T, residual=w.residual)
            oc.append(0, raw_k[b:b + 1, :, h:h + 1], raw_v[b:b + 1, :, h:h + 1])
            qv = q[b:b + 1, h * hg:(h + 1) * hg].float().numpy()
            oc.decode(0, qv)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    byts = decode_bytes(one, T) * done
    return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {len(units)} (sequence, KV head) units of one layer at "
                      f"{T} tokens: oracle quantise + fp64 dequantise + fp64 attention, "
                      f"{dt:.1f} s on one host thread"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--workload", default="kivi2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the hot path shards "
              "by (sequence, KV head) with no communication, so more GPUs only repeat the "
              "one-GPU kernel on their own cache slabs", file=sys.stderr)
        sys.exit(2)
    w = synth.WORKLOADS[args.workload]
    if w.scheme != synth.KIVI:
        sys.exit("bench.py times the KIVI workloads")
    r = gpu_bench(args, w)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: KIVI {w.bits}-bit cache, {args.layers} layers of "
                        f"Llama-3-8B layer shape ({w.q_heads}q/{w.kv_heads}kv heads, head_dim "
                        f"{w.head_dim}), batch {w.batch}, context {w.tokens}+, residual "
                        f"{w.residual} bf16 tokens; step = append 1 token + decode, every layer",
            "layers": args.layers, "global_batch": w.batch, "seq_len": w.tokens,
            "bits": w.bits, "group": 32, "residual": w.residual, "parallelism": "none (1 GPU)",
        },
        "pct_of_hbm_peak": round(100 * r["gbs"] / HBM_PEAK_GBS, 2),
        "append_tokens_per_s": round(r["append_tps"]),
        "append_prefill_gbs": round(r["prefill_gbs"], 1),
        "roofline": r["roofline"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
