"""CPU oracle for the quantised KV cache -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

A plain, slow, obviously correct statement of what the hot path computes,
written from the pages on KV-cache quantisation:

  * "Quantising the Cache." (llm.curionode.com, kv-quantisation): Workshop
    (symmetric round-to-nearest per head per token; Llama 3 8B concurrency),
    "Twice the users for nearly nothing", Terms.
  * "Quantizing the KV cache" (learning.iampt.xyz/quantization/kv-cache):
    "The other big memory user" (KV-bytes equation), "How the KV cache is
    quantized" (FP8 cache with per-head scales), "Keys and values are shaped
    differently" (per-channel keys, per-token values, window of recent tokens),
    going deeper (the Q_b formula, "Why values per token").
  * "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
    (crackai.dev): How It Works (residual length of recent tokens).
  * "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
    Quantization" (research.elamur.ai): Summary (keys quantised before RoPE).
  * "kv cache quantization" glossary (chipfoundryservices.com): The KV Cache
    Problem (LLaMA-7B bytes per token).

Encodings are reproduced bit-exactly in float32 (numpy float32 arrays: IEEE
single operations, correctly rounded division, no fused multiply-add, no
flush-to-zero); attention is computed by its definition in float64.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP library
and imports nothing from it.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, invariants or brute force; none is
"parity unpinned" except the qualitative accuracy claims listed in
``accuracy_claims_unpinned``.
"""

from . import accounting, codec, rope, attention, layout, cache  # noqa: F401

# Claims on the pages that need trained models or datasets absent here; the
# oracle makes no statement about them (parity unpinned).
accuracy_claims_unpinned = (
    "micro's held-out loss increase per cache bit width (Quantising the Cache.)",
    "KIVI < 0.1 perplexity at 2 bits; KVQuant perplexity on Wikitext-2 / C4",
    "per-token 48% vs per-channel 16% relative error on the page's 24x16 slice",
)
