"""Benchmark of the quantised-KV-cache hot path on one MI355X.

A step is one decode step of a 32-layer model of Llama-3-8B layer shape
(32 query / 8 KV heads, head_dim 128) at batch 16 over a KIVI 2-bit cache with
a 128-token bf16 residual window: for every layer, quantize-append of the new
token of each sequence (flushing a 32-token group whenever the window fills),
then decode attention of one query per sequence over all cached tokens -- one
kvq_append_decode call per layer, a single launch on the steps whose token
lands in the residual window. The
32 layers have distinct caches (about 2 GB, far beyond the 256 MB Infinity
Cache), so every decode reads its cache from HBM. The context starts at 4096
tokens (the workload's size) and grows by one token per step.

value = algorithmic bytes of the K timed steps / their wall time (GB/s):
decode reads the packed codes, fp32 scales/offsets, the residual ring, the
query and writes the output; append reads the new K/V rows and writes the ring
(and, on flush steps, reads 32 ring rows and writes the page).

Also reported: quantize-append tokens/s for the 4096-token prefill of each
layer, the decode kernel against the HBM roofline, and the CPU oracle on a
bounded sample.

Roofline: the decode kernel's algorithmic bytes per launch (the bytes a decode
call must move: packed codes, scales and offsets of every page, the residual
rows, the query and the output) divided by its launch duration. After the
timed steps every layer is filled up to a fixed context (the workload's 4096
tokens + 64), so the roofline launch is the same whatever --steps and --warmup
are (up to 64 together); bursts of back-to-back decode launches over the 32
layers run for at least --roofline-ms, each burst between HIP events recorded
on the launch stream (no host launch latency is counted), and the mean, median
and minimum per launch are reported. `--copy-calibration` runs only a plain
device-to-device copy of 256 MiB, whose hardware FETCH_SIZE/WRITE_SIZE
counters calibrate the decode kernel's counter readings into HBM bytes.

Per-workload rows: prefill quantize-append tokens/s, the one-token append and
the decode of each of the five workloads at full size (tiny, kivi2, fp8, int4,
longctx), each decode against the HBM roofline.

CPU baseline: the oracle, on a pool of host processes forked before the first
GPU call, one per host core of this process's CPU share (at most 16), each on
its own whole (sequence, KV head) units of the workload for a bounded time.
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

# Hardware byte counters of the decode kernel (rocprofv3 --pmc, FETCH_SIZE and
# WRITE_SIZE in separate runs of `bench.py --gpus 1 --steps 20 --warmup 5`;
# median KiB per dispatch of the roofline launches at the fixed context), with
# the scale that turns each counter into bytes: a plain 256 MiB device copy
# (`--copy-calibration`) reads FETCH_SIZE = 131084 KiB for 262144 KiB read and
# WRITE_SIZE = 262144 KiB for 262144 KiB written. The readings hold only for the
# kernel sources they were taken with (SHA-256 over DECODE_SOURCES); after any
# change to those, `traffic` is reported as null until they are taken again.
ROOFLINE_EXTRA = 64            # roofline context = workload tokens + this
COUNTERS = {
    "kivi2": {"context": 4096 + ROOFLINE_EXTRA, "fetch_kib": 30747.38, "write_kib": 904.25,
              "fetch_scale": 262144 / 131084, "write_scale": 1.0,
              "sources_sha256": "eca54787c857f4fd22490c3a1cb4c558b15b44c089421ce8c3ed9af0173859b6"},
}
DECODE_SOURCES = ["decode_mfma.hip", "kvq_device.h", "kvq_internal.h", "kvq_merge.h", "kvq_wave.h"]


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_quantisation_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(w, context):
    """HBM bytes per decode launch from the stored counter readings, or None."""
    c = COUNTERS.get(w.name)
    if (not c or c["fetch_kib"] is None or c["context"] != context
            or c["sources_sha256"] != decode_sources_sha256()):
        return None
    return round((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024)
METRIC = "decode-attn effective HBM GB/s (% of MI355X peak) + quantize-append tokens/s"


def kivi_q(T, R):
    return 32 * (max(0, T - R) // 32)


def kivi_page_bytes(w):
    """Bytes of one KIVI page: key codes, value codes (v_bits when set), fp32
    scale and offset per key channel and per value token."""
    vb = w.v_bits or w.bits
    return 32 * w.head_dim * (w.bits + vb) // 8 + 8 * w.head_dim + 256


def decode_bytes(w, T, in_bytes=2, q_bytes=2):
    """Algorithmic bytes of one decode call over T tokens (all sequences/heads)."""
    page = kivi_page_bytes(w)
    q = kivi_q(T, w.residual)
    per_unit = (q // 32) * page + (T - q) * 2 * w.head_dim * in_bytes
    hg = w.q_heads // w.kv_heads
    per_unit += hg * w.head_dim * (q_bytes + 4)
    return w.batch * w.kv_heads * per_unit


def ragged_decode_bytes(w, lens, in_bytes=2, q_bytes=2):
    """Algorithmic bytes of a ragged decode where sequence b holds lens[b]
    tokens (its own fill level): its q(T_b) / 32 pages, its T_b - q(T_b) ring
    rows, the query and the output."""
    page = kivi_page_bytes(w)
    hg = w.q_heads // w.kv_heads
    total = 0
    for Tb in lens:
        q = kivi_q(Tb, w.residual)
        per_unit = (q // 32) * page + (Tb - q) * 2 * w.head_dim * in_bytes
        total += w.kv_heads * (per_unit + hg * w.head_dim * (q_bytes + 4))
    return total


def append_bytes(w, T_old, n, in_bytes=2):
    """Algorithmic bytes of appending n tokens to a T_old-token KIVI cache."""
    d, R = w.head_dim, w.residual
    page = kivi_page_bytes(w)
    q0, q1 = kivi_q(T_old, R), kivi_q(T_old + n, R)
    row = 2 * d * in_bytes                         # one K row + one V row
    rd = n * row                                   # new tokens
    from_ring = max(0, min(q1, T_old) - q0)        # flushed tokens that sat in the ring
    rd += from_ring * row
    wr = ((q1 - q0) // 32) * page + max(0, T_old + n - max(q1, T_old)) * row
    return w.batch * w.kv_heads * (rd + wr)


def token_bytes(w):
    """Cache bytes per token per KV head (codes + fp32 metadata) of a
    non-KIVI scheme."""
    d, b = w.head_dim, w.bits
    if w.scheme == synth.SYM_TOKEN:
        return 2 * (d * b // 8 + 4)
    if w.scheme == synth.BF16_CACHE:
        return 4 * d
    return 2 * d   # FP8: one byte per value, per-head scales are arguments


def any_decode_bytes(w, T):
    """Algorithmic bytes of one decode call for any scheme."""
    in_b = 2 if w.in_dtype == torch.bfloat16 else 4
    q_b = 2 if w.q_dtype == torch.bfloat16 else 4
    if w.scheme == synth.KIVI:
        return decode_bytes(w, T, in_b, q_b)
    hg = w.q_heads // w.kv_heads
    return w.batch * w.kv_heads * (T * token_bytes(w) + hg * w.head_dim * (q_b + 4))


def any_append_bytes(w, T_old, n):
    """Algorithmic bytes of appending n tokens for any scheme."""
    in_b = 2 if w.in_dtype == torch.bfloat16 else 4
    if w.scheme == synth.KIVI:
        return append_bytes(w, T_old, n, in_b)
    return w.batch * w.kv_heads * n * (2 * w.head_dim * in_b + token_bytes(w))


def bf16_baseline_decode_us(w, reps=5, tokens=None):
    """Decode time of the unquantised bfloat16 cache (KVQ_BF16_CACHE) at the
    shape of workload `w` (same batch, heads, head_dim and context, or
    `tokens`; no rotation): the same-GPU baseline the quantised caches are
    compared to."""
    dev = torch.device("cuda", 0)
    T = tokens or w.tokens
    wb = synth.scaled(w, scheme=synth.BF16_CACHE, bits=16, residual=0, rope_theta=0.0,
                      in_dtype=torch.bfloat16, q_dtype=torch.bfloat16, tokens=T)
    cfg = kvq.make_config(kvq.KVQ_BF16_CACHE, 16, 1, w.q_heads, w.kv_heads, w.head_dim, w.batch,
                          T + 1)
    cache = kvq.alloc_cache(cfg, device=dev, zero=False)
    k, v = synth.keys_values(wb, device=dev)
    kvq.kvq_quantize_append(cfg, cache, 0, 0, T, k, v)
    del k, v
    q = synth.query(wb, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = kvq.alloc_workspace(cfg, T, device=dev)
    stream = torch.cuda.current_stream()
    kvq.kvq_decode_attention(cfg, cache, 0, T, q, out, ws, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        kvq.kvq_decode_attention(cfg, cache, 0, T, q, out, ws, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    del cache
    torch.cuda.empty_cache()
    return a.elapsed_time(b) * 1e3 / reps


def workload_kernels(name, reps=5):
    """Times the path's kernels on one workload at its full size: the prefill
    quantize-append (one call for the whole context), the 1-token append, and
    decode over the full context (back-to-back launches between HIP events)."""
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[name]
    T = w.tokens
    dt = {torch.bfloat16: kvq.KVQ_BF16, torch.float32: kvq.KVQ_F32}
    cfg = kvq.make_config(w.scheme, w.bits, 1, w.q_heads, w.kv_heads, w.head_dim, w.batch, T + 1,
                          v_bits=w.v_bits,
                          residual=w.residual, in_dtype=dt[w.in_dtype], q_dtype=dt[w.q_dtype],
                          rope_theta=w.rope_theta)
    cache = kvq.alloc_cache(cfg, device=dev, zero=False)
    k, v = synth.keys_values(w, device=dev)
    ks = vs = None
    if w.scheme == synth.FP8_E4M3:
        ks, vs = synth.fp8_scales(k, v)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    pre_us = timed(lambda: kvq.kvq_quantize_append(cfg, cache, 0, 0, T, k, v, ks, vs, stream=stream),
                   reps)
    del k, v
    k1, v1 = synth.keys_values(w, tokens=1, device=dev, tag=1)
    app_us = timed(lambda: kvq.kvq_quantize_append(cfg, cache, 0, T, 1, k1, v1, ks, vs,
                                                   stream=stream), reps)
    q = synth.query(w, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = kvq.alloc_workspace(cfg, T + 1, device=dev)
    dec_us = timed(lambda: kvq.kvq_decode_attention(cfg, cache, 0, T + 1, q, out, ws, k_scale=ks,
                                                    v_scale=vs,
                                                    stream=stream), reps)
    pre_b, app_b, dec_b = any_append_bytes(w, 0, T), any_append_bytes(w, T, 1), \
        any_decode_bytes(w, T + 1)
    del cache, ws
    torch.cuda.empty_cache()
    base = {}
    if w.scheme in (synth.KIVI, synth.FP8_E4M3) and w.rope_theta == 0.0:
        bus = bf16_baseline_decode_us(w, reps)
        base = {"bf16_cache_decode_us": round(bus, 2),
                "decode_speedup_vs_bf16_cache": round(bus / dec_us, 2)}
    return {
        "workload": name, "batch": w.batch, "context": T, "bits": w.bits,
        "v_bits": w.v_bits or w.bits,
        "prefill_us": round(pre_us, 2), "prefill_gbs": round(pre_b / pre_us / 1e3, 1),
        "prefill_tokens_per_s": round(w.batch * T / (pre_us * 1e-6)),
        "append1_us": round(app_us, 2), "append1_gbs": round(app_b / app_us / 1e3, 1),
        "decode_us": round(dec_us, 2), "decode_gbs": round(dec_b / dec_us / 1e3, 1),
        "decode_frac_of_hbm_peak": round(dec_b / dec_us / 1e3 / HBM_PEAK_GBS, 4),
        "decode_bytes": dec_b, "prefill_bytes": pre_b, **base,
    }


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

    # per-layer inputs of the decode steps (and of the fill up to the roofline context)
    n_new = max(W + K, ROOFLINE_EXTRA)
    news = [synth.keys_values(w, layer=layer, tokens=n_new, device=dev, tag=1) for layer in range(L)]
    qs = [synth.query(w, layer=layer, device=dev) for layer in range(L)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device=dev) for q in qs]

    # one contiguous [B, 1, H, d] tensor per (layer, step), made before timing
    news = [(kn.unbind(1), vn.unbind(1)) for kn, vn in news]
    news = [([x.unsqueeze(1).contiguous() for x in kl], [x.unsqueeze(1).contiguous() for x in vl])
            for kl, vl in news]

    def step(i):
        # every layer: append the step's token, then decode over all tokens
        # (kvq_append_decode: one launch when the token lands in the ring, the
        # append's kernels first on the steps that encode a page)
        T = T0 + i
        for layer in range(L):
            kvq.kvq_append_decode(cfg, cache, layer, T, news[layer][0][i], news[layer][1][i],
                                  qs[layer], outs[layer], ws, stream=stream)

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

    # decode kernel alone, at a fixed context: every layer is filled up to
    # T0 + ROOFLINE_EXTRA tokens (whatever the step counts were), then bursts
    # of back-to-back launches over the 32 layers, each burst between HIP
    # events on the launch stream, for at least roofline_ms
    T_end = T0 + max(W + K, ROOFLINE_EXTRA)
    for i in range(W + K, T_end - T0):
        for layer in range(L):
            kvq.kvq_quantize_append(cfg, cache, layer, T0 + i, 1, news[layer][0][i],
                                    news[layer][1][i], stream=stream)
    for layer in range(L):   # warm the launch path at this context length
        kvq.kvq_decode_attention(cfg, cache, layer, T_end, qs[layer], outs[layer], ws, stream=stream)
    torch.cuda.synchronize()
    burst_us = []
    spent = 0.0
    while spent < args.roofline_ms * 1e-3 or len(burst_us) < 8:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(32)]
        for a, b in evs:
            a.record(stream)
            for layer in range(L):
                kvq.kvq_decode_attention(cfg, cache, layer, T_end, qs[layer], outs[layer], ws,
                                         stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        for a, b in evs:
            us = a.elapsed_time(b) * 1e3 / L
            burst_us.append(us)
            spent += us * L * 1e-6
    burst_us.sort()
    avg_us = sum(burst_us) / len(burst_us)
    med_us = burst_us[len(burst_us) // 2]
    min_us = burst_us[0]
    n_rep = 4
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = graph_replay(cfg, cache, ws, qs, outs, news, L, T_end, n_rep)
    cache_bytes = int(cache.numel())

    # several causal queries per sequence over the same caches: 4 and 8
    # (e.g. speculated tokens being verified; their tokens in the ring) on the
    # kernel of four queries per block, whose keys are dequantised once per
    # page for the four, and a chunk of 64 (chunked prefill; tokens reaching
    # into the pages) on the kernel of 32 queries per block, which copies and
    # dequantises each 32-token chunk once for the 32
    multi = []
    for nq in (4, 8, 64):
        qm = [torch.stack([synth.query(w, layer=l, device=dev, tag=1 + i) for i in range(nq)], dim=1)
              .contiguous() for l in range(L)]
        om = [torch.empty(x.shape, dtype=torch.float32, device=dev) for x in qm]
        wsm = torch.zeros(nq * kvq.kvq_cache_bytes(cfg, T_end, kvq.KVQ_BYTES_WORKSPACE),
                          dtype=torch.uint8, device=dev)
        reps = []
        for rep in range(4):   # the first pass warms up; the median of three timed
            a.record(stream)
            for layer in range(L):
                kvq.kvq_decode_attention_multi(cfg, cache, layer, T_end, qm[layer], om[layer], wsm,
                                               stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            if rep:
                reps.append(a.elapsed_time(b) * 1e3 / L)
        multi_us = sorted(reps)[1]
        multi_b = decode_bytes(w, T_end) + (nq - 1) * w.batch * w.q_heads * w.head_dim * (2 + 4)
        multi.append({"n_queries": nq, "median_launch_us": round(multi_us, 3), "bytes_per_launch": multi_b,
                      "gbs": round(multi_b / (multi_us * 1e-6) / 1e9, 1),
                      "x_one_query": round(multi_us / burst_us[len(burst_us) // 2], 2),
                      "kernel": ("kivi_chunk_kernel<2> (rows b * n_q / 32 + i, one split)" if nq % 32 == 0
                                 else "kivi_deq_kernel<2,2,128> (rows b * n_q / 4 + i, merge fused)")})
        del qm, om, wsm

    # ragged batch: 32 more layer caches whose sequences hold lens[b] tokens
    # each (filled by one ragged quantize-append per layer), lens uniform in
    # [T/2, T] (seeded); decode each sequence over its own fill level
    del cache
    torch.cuda.empty_cache()
    gen = torch.Generator().manual_seed(0)
    lens = torch.randint(T_end // 2, T_end + 1, (w.batch,), generator=gen).tolist()
    seq = torch.tensor(lens, dtype=torch.int64, device=dev)
    zeros = torch.zeros(w.batch, dtype=torch.int64, device=dev)
    rcache = kvq.alloc_cache(cfg, device=dev, zero=False)
    for layer in range(L):
        k, v = synth.keys_values(w, layer=layer, tokens=T_end, device=dev)
        kvq.kvq_quantize_append_ragged(cfg, rcache, layer, zeros, seq, k, v, stream=stream)
        del k, v
    for layer in range(L):
        kvq.kvq_decode_attention_ragged(cfg, rcache, layer, T_end, seq, qs[layer], outs[layer], ws,
                                        stream=stream)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n_rep):
        for layer in range(L):
            kvq.kvq_decode_attention_ragged(cfg, rcache, layer, T_end, seq, qs[layer], outs[layer],
                                            ws, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    ragged_us = a.elapsed_time(b) * 1e3 / (n_rep * L)
    ragged_b = ragged_decode_bytes(w, lens)
    del rcache
    ragged = {"avg_launch_us": round(ragged_us, 3), "bytes_per_launch": ragged_b,
              "gbs": round(ragged_b / (ragged_us * 1e-6) / 1e9, 1),
              "lengths": f"per sequence uniform in [{T_end // 2}, {T_end}] (seed 0); "
                         f"mean {sum(lens) / len(lens):.0f}"}
    per_launch = decode_bytes(w, T_end)
    achieved = per_launch / (avg_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(w, T_end),
                "kernel": f"kivi_mfma_kernel<{w.bits},{w.v_bits or w.bits},{w.head_dim},"
                          f"{w.q_heads // w.kv_heads}> (decode, merge fused)",
                "avg_launch_us": round(avg_us, 3), "median_launch_us": round(med_us, 3),
                "min_launch_us": round(min_us, 3),
                "frac_at_median": round(per_launch / (med_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "launches": len(burst_us) * L,
                "timed_ms": round(sum(burst_us) * L * 1e-3, 1),
                "bytes_per_launch": per_launch, "context": T_end}
    return {
        "ms_per_step": total_ms / K, "gbs": gbs, "append_tps": append_tps,
        "prefill_ms_per_layer": prefill_ms, "prefill_gbs": prefill_bytes / (prefill_ms * 1e-3) / 1e9,
        "roofline": roofline, "cache_bytes": cache_bytes, "graph": graph,
        "ragged": ragged, "multi": multi,
    }


def graph_replay(cfg, cache, ws, qs, outs, news, L, T, n_rep):
    """The decode burst at a fixed context T and one whole step (append +
    decode, every layer) captured once each in a HIP graph and replayed, so
    no host launch cost is counted. The step appends token T - 2 and decodes
    over T - 1 tokens, a position where no page is encoded (as on the eager
    steps). Replays repeat identical work (the append writes the same ring
    slot with the same row), and their outputs are checked bit for bit
    against eager launches before and after the timed replays."""
    stream = torch.cuda.current_stream()
    # the cache's tokens T - 2 and T - 1: the rows the step and the prefix re-append
    for layer in range(L):
        kvq.kvq_quantize_append(cfg, cache, layer, T - 2, 1, news[layer][0][1], news[layer][1][1],
                                stream=stream)
        kvq.kvq_quantize_append(cfg, cache, layer, T - 1, 1, news[layer][0][0], news[layer][1][0],
                                stream=stream)
    outs_step = [torch.empty_like(o) for o in outs]
    for layer in range(L):
        kvq.kvq_decode_attention(cfg, cache, layer, T, qs[layer], outs[layer], ws, stream=stream)
        kvq.kvq_decode_attention(cfg, cache, layer, T - 1, qs[layer], outs_step[layer], ws, stream=stream)
    torch.cuda.synchronize()
    eager = {"decode_burst": [o.clone() for o in outs], "step": [o.clone() for o in outs_step]}
    target = {"decode_burst": outs, "step": outs_step}

    def burst():
        for layer in range(L):
            kvq.kvq_decode_attention(cfg, cache, layer, T, qs[layer], outs[layer], ws)

    def step():
        for layer in range(L):
            kvq.kvq_append_decode(cfg, cache, layer, T - 2, news[layer][0][1], news[layer][1][1],
                                  qs[layer], outs_step[layer], ws)

    res, ok = {}, True
    for name, fn in (("decode_burst", burst), ("step", step)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for o in target[name]:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        ok &= all(torch.equal(o, e) for o, e in zip(target[name], eager[name]))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_rep):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ok &= all(torch.equal(o, e) for o, e in zip(target[name], eager[name]))
        res[name] = a.elapsed_time(b) * 1e3 / n_rep
        del g
    burst()   # eager again after the replays
    torch.cuda.synchronize()
    ok &= all(torch.equal(o, e) for o, e in zip(outs, eager["decode_burst"]))
    return {"decode_us_per_launch": round(res["decode_burst"] / L, 3),
            "ms_per_step": round(res["step"] / 1e3, 4), "context": T, "step_context": T - 1,
            "outputs_match_eager": ok}


def copy_ceiling(gib=1, reps=10):
    """GB/s of a plain device copy (torch.mul(x, 1.0, out=y): read + write), a
    practical ceiling for streaming kernels on this GPU."""
    dev = torch.device("cuda", 0)
    n = gib * (1 << 30) // 4
    x = torch.randn(n, device=dev)
    y = torch.empty_like(x)
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del x, y
    return round(2 * n * 4 / us / 1e3, 1)


def _oracle_units(job):
    """Worker of the CPU baseline (a process of the pool): the oracle on whole
    (sequence, KV head) units of the workload, layer after layer from `first`
    in steps of `stride`, until `budget_s` seconds of oracle time. Returns
    (units, algorithmic decode bytes of those units, oracle seconds)."""
    name, first, stride, layers, budget_s = job
    import numpy as np
    from oracle.cache import OracleCache
    from threadpoolctl import threadpool_limits
    torch.set_num_threads(1)
    w = synth.WORKLOADS[name]
    hg = w.q_heads // w.kv_heads
    T = w.tokens
    one = synth.scaled(w, batch=1, kv_heads=1, q_heads=hg)
    done, spent = 0, 0.0
    with threadpool_limits(limits=1):
        for layer in range(first, layers, stride):
            k, v = synth.keys_values(w, layer=layer, device="cpu")
            q = synth.query(w, layer=layer, device="cpu")
            raw_k = k.view(torch.int16).numpy().view(np.uint16)
            raw_v = v.view(torch.int16).numpy().view(np.uint16)
            for b in range(w.batch):
                for h in range(w.kv_heads):
                    qv = q[b:b + 1, h * hg:(h + 1) * hg].float().numpy()
                    t0 = time.perf_counter()
                    oc = OracleCache(w.scheme, w.bits, 1, 1, 1, w.head_dim, T, residual=w.residual)
                    oc.append(0, raw_k[b:b + 1, :, h:h + 1], raw_v[b:b + 1, :, h:h + 1])
                    oc.decode(0, qv)
                    spent += time.perf_counter() - t0
                    done += 1
                    if spent > budget_s:
                        return done, decode_bytes(one, T) * done, spent
            del k, v
    return done, decode_bytes(one, T) * done, spent


def host_cpu():
    """(cores this process may run on, capped at the 16 of a one-GPU share;
    CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return min(n, 16), n, model


def cpu_pool():
    """A pool of host processes for the oracle, forked before any GPU call
    (and before torch runs any CPU op), one per usable core."""
    import multiprocessing as mp
    cores, _, _ = host_cpu()
    return mp.get_context("fork").Pool(cores), cores


def cpu_baseline(pool, cores, w, budget_s=12.0):
    """The oracle (as it stands: numpy, fp64 attention) on a bounded sample of
    the workload, in parallel on `cores` host processes: each takes whole
    (sequence, KV head) units -- quantise, dequantise and attend -- of its own
    layers for about budget_s seconds. value = the sum of the processes'
    rates (algorithmic decode bytes of their units / their oracle time)."""
    # process i takes layers i, i + cores, ... (synthetic layers beyond the
    # model's 32 are drawn the same way) until its budget is spent
    jobs = [(w.name, i, cores, 1 << 20, budget_s) for i in range(cores)]
    res = pool.map(_oracle_units, jobs)
    units = sum(r[0] for r in res)
    rate = sum(r[1] / r[2] for r in res if r[2] > 0)
    _, avail, model = host_cpu()
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "host_cores_available": avail, "cpu_model": model,
            "sample": f"{units} (sequence, KV head) units of {w.name} at {w.tokens} tokens, "
                      f"{cores} processes x ~{budget_s:.0f} s of oracle time (numpy, one thread "
                      f"each): quantise + fp64 dequantise + fp64 attention per unit; value = "
                      f"sum over processes of algorithmic decode bytes / oracle time"}


def config_row(name, dec_reps=20, pre_reps=3):
    """One workload at full size on its own cache: prefill quantize-append of
    the whole context (one call), the one-token append, and the decode over
    context + 1 tokens, each launch timed between HIP events on the launch
    stream (median and minimum)."""
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[name]
    T = w.tokens
    dt = {torch.bfloat16: kvq.KVQ_BF16, torch.float32: kvq.KVQ_F32}
    cfg = kvq.make_config(w.scheme, w.bits, 1, w.q_heads, w.kv_heads, w.head_dim, w.batch, T + 1,
                          v_bits=w.v_bits, residual=w.residual, in_dtype=dt[w.in_dtype],
                          q_dtype=dt[w.q_dtype], rope_theta=w.rope_theta)
    cache = kvq.alloc_cache(cfg, device=dev, zero=False)
    k, v = synth.keys_values(w, device=dev)
    ks = vs = None
    if w.scheme == synth.FP8_E4M3:
        ks, vs = synth.fp8_scales(k, v)
    stream = torch.cuda.current_stream()

    def each(fn, n):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) * 1e3 for a, b in evs)

    pre = each(lambda: kvq.kvq_quantize_append(cfg, cache, 0, 0, T, k, v, ks, vs, stream=stream),
               pre_reps)
    del k, v
    k1, v1 = synth.keys_values(w, tokens=1, device=dev, tag=1)
    app = each(lambda: kvq.kvq_quantize_append(cfg, cache, 0, T, 1, k1, v1, ks, vs, stream=stream),
               dec_reps)
    q = synth.query(w, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = kvq.alloc_workspace(cfg, T + 1, device=dev)
    dec = each(lambda: kvq.kvq_decode_attention(cfg, cache, 0, T + 1, q, out, ws, k_scale=ks,
                                                v_scale=vs, stream=stream), dec_reps)
    # four causal queries per sequence over the same cache (the last four
    # tokens' positions; e.g. speculated tokens being verified)
    qm = torch.stack([synth.query(w, device=dev, tag=1 + i) for i in range(4)], dim=1).contiguous()
    om = torch.empty(qm.shape, dtype=torch.float32, device=dev)
    wsm = torch.zeros(4 * kvq.kvq_cache_bytes(cfg, T + 1, kvq.KVQ_BYTES_WORKSPACE), dtype=torch.uint8,
                      device=dev)
    dec4 = each(lambda: kvq.kvq_decode_attention_multi(cfg, cache, 0, T + 1, qm, om, wsm, k_scale=ks,
                                                       v_scale=vs, stream=stream), max(3, dec_reps // 4))
    del cache, ws, wsm
    torch.cuda.empty_cache()
    med = lambda xs: xs[len(xs) // 2]   # noqa: E731
    dec_b, pre_b = any_decode_bytes(w, T + 1), any_append_bytes(w, 0, T)
    return {
        "workload": name, "batch": w.batch, "context": T + 1, "bits": w.bits,
        "kernel": decode_kernel_name(w),
        "decode_us_median": round(med(dec), 2), "decode_us_min": round(dec[0], 2),
        "decode_bytes": dec_b, "decode_gbs": round(dec_b / med(dec) / 1e3, 1),
        "decode_frac_of_hbm_peak": round(dec_b / med(dec) / 1e3 / HBM_PEAK_GBS, 4),
        "prefill_us_median": round(med(pre), 2), "prefill_bytes": pre_b,
        "prefill_tokens_per_s": round(w.batch * T / (med(pre) * 1e-6)),
        "prefill_frac_of_hbm_peak": round(pre_b / med(pre) / 1e3 / HBM_PEAK_GBS, 4),
        "append1_us_median": round(med(app), 2),
        "decode_4_queries_us_median": round(med(dec4), 2),
        "decode_4_queries_x_one_query": round(med(dec4) / med(dec), 2),
    }


def decode_kernel_name(w):
    """The decode kernel the library runs for workload w (for reading profiles)."""
    hg = w.q_heads // w.kv_heads
    if w.scheme == synth.KIVI and w.rope_theta > 0:
        return f"rope4_kernel<{w.head_dim},4>" if hg == 4 else \
            f"kivi_mfma_kernel<2,2,{w.head_dim},{hg},true>"
    if w.scheme == synth.KIVI and w.bits in (2, 4) and w.in_dtype == torch.bfloat16:
        return f"kivi_mfma_kernel<{w.bits},{w.v_bits or w.bits},{w.head_dim},{hg},false>"
    if w.scheme == synth.FP8_E4M3 and w.rope_theta == 0:
        return f"paged_mfma_kernel<FP8_E4M3,{w.head_dim},{hg}>"
    if (w.scheme == synth.SYM_TOKEN and w.rope_theta == 0 and w.bits in (2, 4, 8)
            and not (w.bits == 2 and w.head_dim == 32)):
        return f"paged_mfma_kernel<SYM_TOKEN,{w.head_dim},{hg},{w.bits},{w.bits}>"
    return f"decode_split_kernel<scheme {w.scheme},{w.bits},{w.head_dim},{hg}>"


def copy_calibration(mib=256, reps=5):
    """A plain device copy of known size, for calibrating the byte counters."""
    dev = torch.device("cuda", 0)
    n = mib * (1 << 20) // 4
    x = torch.randn(n, device=dev)
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--workload", default="kivi2")
    ap.add_argument("--roofline-ms", type=float, default=200.0,
                    help="minimum time of the roofline decode bursts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload rows")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--workload-kernels", nargs="*", metavar="NAME",
                    help="only time prefill, 1-token append and decode of the named "
                         "workloads at full size (one JSON line each)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the hot path shards "
              "by (sequence, KV head) with no communication, so more GPUs only repeat the "
              "one-GPU kernel on their own cache slabs", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload_kernels is not None:
        for name in args.workload_kernels or list(synth.WORKLOADS):
            print(json.dumps(workload_kernels(name)), flush=True)
            torch.cuda.empty_cache()
        return
    w = synth.WORKLOADS[args.workload]
    if w.scheme != synth.KIVI:
        sys.exit("bench.py times the KIVI workloads")
    # the oracle's process pool is forked before anything touches the GPU
    pool, cores = (None, 0) if args.no_cpu_baseline else cpu_pool()
    r = gpu_bench(args, w)
    base_us = bf16_baseline_decode_us(w, tokens=r["roofline"]["context"])
    rows = []
    if not args.no_configs:
        ro = r["roofline"]
        rows.append({
            "workload": w.name, "batch": w.batch, "context": ro["context"], "bits": w.bits,
            "kernel": decode_kernel_name(w), "layers": args.layers,
            "decode_us_median": ro["median_launch_us"], "decode_us_min": ro["min_launch_us"],
            "decode_bytes": ro["bytes_per_launch"],
            "decode_gbs": round(ro["bytes_per_launch"] / ro["median_launch_us"] / 1e3, 1),
            "decode_frac_of_hbm_peak": ro["frac_at_median"],
            "prefill_us_median": round(r["prefill_ms_per_layer"] * 1e3, 2),
            "prefill_tokens_per_s": round(r["append_tps"]),
            "prefill_frac_of_hbm_peak": round(r["prefill_gbs"] / HBM_PEAK_GBS, 4),
            "note": "decode rotates over the 32 layer caches (2 GB, beyond the 256 MB "
                    "Infinity Cache)"})
        for name in ("tiny", "fp8", "int4", "longctx"):
            rows.append(config_row(name))
            torch.cuda.empty_cache()
    cpu = None
    if pool is not None:
        cpu = cpu_baseline(pool, cores, w)
        pool.close()
        pool.join()
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
        "dtype": "u2 codes; f16/bf16 mfma, f32 accumulate",
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
        "workloads": rows,
        "graph_replay": r["graph"],
        "ragged_decode": r["ragged"],
        "multi_query_decode": r["multi"],
        "bf16_cache_baseline": {
            "decode_us": round(base_us, 3), "context": r["roofline"]["context"],
            "speedup_of_quantised_decode": round(base_us / r["roofline"]["avg_launch_us"], 2),
            "note": "same shape, unquantised bfloat16 cache (KVQ_BF16_CACHE) on the same GPU; "
                    "KVQuant reports 1.2-1.6x (K) and 1.3-1.7x (V) for 4-bit vs fp16 on an A6000 "
                    "(other GPU, context only)"},
        "copy_ceiling_gbs": copy_ceiling(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
