"""kvq: quantised KV cache for MI355X (gfx950).

The product is libkvq.so (C ABI in include/kvq.h, HIP kernels in csrc/);
``kvq`` is its thin ctypes binding with the same entry-point names.
"""

from .kvq import (  # noqa: F401
    KVQ_BF16, KVQ_BYTES_CACHE, KVQ_BYTES_FORMULA, KVQ_BYTES_WORKSPACE, KVQ_ERR_CAPACITY,
    KVQ_ERR_DEVICE, KVQ_ERR_INVALID, KVQ_ERR_NULL, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE,
    KVQ_BF16_CACHE, KVQ_F32, KVQ_FP8_E4M3, KVQ_FP8_E5M2, KVQ_FP8K_SYMV, KVQ_FP8K_KIVIV, KVQ_KIVI, KVQ_OK,
    KVQ_SYM_TOKEN, KvqError, alloc_cache,
    alloc_workspace, kvq_abi_version, kvq_cache_bytes, kvq_config, kvq_decode_attention,
    kvq_decode_attention_multi, kvq_decode_attention_noalloc, kvq_decode_attention_ragged,
    kvq_quantize_append_ragged, KVQ_NOALLOC_SCRATCH_BYTES, kvq_paged_cache_bytes,
    kvq_quantize_append_paged, kvq_decode_attention_paged, kvq_append_decode,
    kvq_quantize_append, lib, make_config, status_string,
)
