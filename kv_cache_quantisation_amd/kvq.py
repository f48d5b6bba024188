"""ctypes binding of libkvq.so -- argument marshalling only.

Each function has the name of the C entry point it calls and forwards plain
pointers and sizes; torch is used for device memory and the current HIP stream
(``torch.cuda.current_stream().cuda_stream`` is PyTorch-ROCm's name for the
hipStream_t). Every computation happens in the library's HIP kernels. There is
no fallback: if libkvq.so is missing or fails to load, every call raises.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_NULL, KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED = 0, -1, -2, -3
KVQ_ERR_CAPACITY, KVQ_ERR_WORKSPACE, KVQ_ERR_DEVICE = -4, -5, -6
KVQ_KIVI, KVQ_SYM_TOKEN, KVQ_FP8_E4M3, KVQ_BF16_CACHE, KVQ_FP8_E5M2, KVQ_FP8K_SYMV, KVQ_FP8K_KIVIV = 0, 1, 2, 3, 4, 5, 6
KVQ_F32, KVQ_BF16 = 0, 1
KVQ_BYTES_FORMULA, KVQ_BYTES_CACHE, KVQ_BYTES_WORKSPACE = 0, 1, 2

ABI_VERSION = 11  # KVQ_ABI_VERSION of include/kvq.h that this binding mirrors

SYMBOLS = ("kvq_cache_bytes", "kvq_quantize_append", "kvq_quantize_append_ragged",
           "kvq_decode_attention", "kvq_decode_attention_ragged", "kvq_decode_attention_multi",
           "kvq_decode_attention_noalloc", "kvq_paged_cache_bytes", "kvq_quantize_append_paged",
           "kvq_decode_attention_paged", "kvq_append_decode", "kvq_status_string",
           "kvq_abi_version")
KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20


class KvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class kvq_config(ctypes.Structure):
    """Mirror of the C struct kvq_config (include/kvq.h)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("scheme", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("layers", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
        ("group", ctypes.c_int32),
        ("residual", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("v_bits", ctypes.c_int32),
        ("outliers", ctypes.c_int32),
    ]


def make_config(scheme, bits, layers, q_heads, kv_heads, head_dim, batch, max_tokens,
                residual=0, in_dtype=KVQ_BF16, q_dtype=KVQ_BF16, rope_theta=0.0,
                sm_scale=0.0, num_splits=0, group=32, v_bits=0, outliers=0):
    c = kvq_config()
    c.struct_size = ctypes.sizeof(kvq_config)
    c.scheme, c.bits, c.layers = scheme, bits, layers
    c.q_heads, c.kv_heads, c.head_dim = q_heads, kv_heads, head_dim
    c.batch, c.max_tokens, c.group, c.residual = batch, max_tokens, group, residual
    c.in_dtype, c.q_dtype = in_dtype, q_dtype
    c.rope_theta, c.sm_scale, c.num_splits = rope_theta, sm_scale, num_splits
    c.v_bits = v_bits
    c.outliers = outliers
    return c


_lib = None


def lib():
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                               "kv_cache_quantisation_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        cfgp = ctypes.POINTER(kvq_config)
        L.kvq_cache_bytes.argtypes = [cfgp, I64, I32]
        L.kvq_cache_bytes.restype = I64
        L.kvq_quantize_append.argtypes = [cfgp, P, I32, I64, I64, P, P, P, P, P]
        L.kvq_quantize_append.restype = I32
        L.kvq_quantize_append_ragged.argtypes = [cfgp, P, I32, P, P, I64, P, P, P, P, P]
        L.kvq_quantize_append_ragged.restype = I32
        L.kvq_decode_attention.argtypes = [cfgp, P, I32, I64, P, P, P, P, P, ctypes.c_size_t, P]
        L.kvq_decode_attention.restype = I32
        L.kvq_decode_attention_ragged.argtypes = [cfgp, P, I32, I64, P, P, P, P, P, P,
                                                  ctypes.c_size_t, P]
        L.kvq_decode_attention_ragged.restype = I32
        L.kvq_decode_attention_multi.argtypes = [cfgp, P, I32, I64, I32, P, P, P, P, P,
                                                 ctypes.c_size_t, P]
        L.kvq_decode_attention_multi.restype = I32
        L.kvq_decode_attention_noalloc.argtypes = [cfgp, P, I32, I64, P, P, P, P, P]
        L.kvq_decode_attention_noalloc.restype = I32
        L.kvq_paged_cache_bytes.argtypes = [cfgp, I64]
        L.kvq_paged_cache_bytes.restype = I64
        L.kvq_quantize_append_paged.argtypes = [cfgp, P, I32, P, I32, I64, P, P, I64, P, P, P, P, P]
        L.kvq_quantize_append_paged.restype = I32
        L.kvq_decode_attention_paged.argtypes = [cfgp, P, I32, P, I32, I64, I64, P, P, P, P, P, P,
                                                 ctypes.c_size_t, P]
        L.kvq_decode_attention_paged.restype = I32
        L.kvq_append_decode.argtypes = [cfgp, P, I32, I64, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.kvq_append_decode.restype = I32
        L.kvq_status_string.argtypes = [I32]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_abi_version.argtypes = []
        L.kvq_abi_version.restype = I32
        if L.kvq_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} reports ABI {L.kvq_abi_version()}, the binding "
                               f"expects {ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


def _ptr(x):
    """Device address of a tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def status_string(status):
    return lib().kvq_status_string(status).decode()


def kvq_abi_version():
    return lib().kvq_abi_version()


def kvq_cache_bytes(cfg, tokens, kind):
    """Byte count for `tokens` tokens per sequence (raises on a negative status)."""
    v = lib().kvq_cache_bytes(ctypes.byref(cfg), tokens, kind)
    if v < 0:
        raise KvqError(v, "kvq_cache_bytes")
    return v


def kvq_quantize_append(cfg, cache, layer, past_tokens, new_tokens, k_new, v_new,
                        k_scale=None, v_scale=None, stream=None, check=True):
    st = lib().kvq_quantize_append(ctypes.byref(cfg), _ptr(cache), layer, past_tokens,
                                   new_tokens, _ptr(k_new), _ptr(v_new), _ptr(k_scale),
                                   _ptr(v_scale), _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_quantize_append")
    return st


def kvq_quantize_append_ragged(cfg, cache, layer, seq_past, seq_new, k_new, v_new, k_scale=None,
                               v_scale=None, stream=None, check=True):
    """seq_past, seq_new: device int64 tensors [batch]; k_new, v_new
    [batch, new_max, kv_heads, head_dim] (sequence b's first seq_new[b] rows)."""
    st = lib().kvq_quantize_append_ragged(ctypes.byref(cfg), _ptr(cache), layer, _ptr(seq_past),
                                          _ptr(seq_new), k_new.shape[1], _ptr(k_new),
                                          _ptr(v_new), _ptr(k_scale), _ptr(v_scale),
                                          _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_quantize_append_ragged")
    return st


def kvq_decode_attention(cfg, cache, layer, tokens, q, out, workspace, workspace_bytes=None,
                         k_scale=None, v_scale=None, stream=None, check=True):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvq_decode_attention(ctypes.byref(cfg), _ptr(cache), layer, tokens, _ptr(q),
                                    _ptr(k_scale), _ptr(v_scale), _ptr(out), _ptr(workspace),
                                    workspace_bytes, _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention")
    return st


def kvq_decode_attention_noalloc(cfg, cache, layer, tokens, q, out, k_scale=None, v_scale=None,
                                 stream=None, check=True):
    """kvq_decode_attention on the library's own scratch array (no workspace)."""
    st = lib().kvq_decode_attention_noalloc(ctypes.byref(cfg), _ptr(cache), layer, tokens, _ptr(q),
                                            _ptr(k_scale), _ptr(v_scale), _ptr(out),
                                            _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention_noalloc")
    return st


def kvq_append_decode(cfg, cache, layer, past_tokens, k_new, v_new, q, out, workspace,
                      workspace_bytes=None, k_scale=None, v_scale=None, stream=None, check=True):
    """One step: append one token per sequence ([batch, 1, kv_heads, head_dim])
    at past_tokens, then decode over past_tokens + 1 tokens."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvq_append_decode(ctypes.byref(cfg), _ptr(cache), layer, past_tokens, _ptr(k_new),
                                 _ptr(v_new), _ptr(k_scale), _ptr(v_scale), _ptr(q), _ptr(out),
                                 _ptr(workspace), workspace_bytes, _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_append_decode")
    return st


def kvq_decode_attention_multi(cfg, cache, layer, tokens, q, out, workspace, workspace_bytes=None,
                               k_scale=None, v_scale=None, stream=None, check=True):
    """q, out: [batch, n_queries, q_heads, head_dim]; query i attends causally to
    tokens [0, tokens - n_queries + i]."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvq_decode_attention_multi(ctypes.byref(cfg), _ptr(cache), layer, tokens,
                                          q.shape[1], _ptr(q), _ptr(k_scale), _ptr(v_scale),
                                          _ptr(out), _ptr(workspace), workspace_bytes,
                                          _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention_multi")
    return st


def kvq_decode_attention_ragged(cfg, cache, layer, tokens, seq_tokens, q, out, workspace,
                                workspace_bytes=None, k_scale=None, v_scale=None, stream=None,
                                check=True):
    """seq_tokens: device int64 tensor [batch] of per-sequence token counts."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvq_decode_attention_ragged(ctypes.byref(cfg), _ptr(cache), layer, tokens,
                                           _ptr(seq_tokens), _ptr(q), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(out), _ptr(workspace),
                                           workspace_bytes, _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention_ragged")
    return st


def kvq_paged_cache_bytes(cfg, num_blocks):
    v = lib().kvq_paged_cache_bytes(ctypes.byref(cfg), num_blocks)
    if v < 0:
        raise KvqError(v, "kvq_paged_cache_bytes")
    return v


def kvq_quantize_append_paged(cfg, cache, layer, block_table, num_blocks, seq_past, seq_new,
                              k_new, v_new, k_scale=None, v_scale=None, stream=None, check=True):
    """block_table: device int32 [batch, max_blocks]; seq_past, seq_new: device
    int64 [batch]; k_new, v_new [batch, new_max, kv_heads, head_dim]."""
    st = lib().kvq_quantize_append_paged(ctypes.byref(cfg), _ptr(cache), layer, _ptr(block_table),
                                         block_table.shape[1], num_blocks, _ptr(seq_past),
                                         _ptr(seq_new), k_new.shape[1], _ptr(k_new), _ptr(v_new),
                                         _ptr(k_scale), _ptr(v_scale), _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_quantize_append_paged")
    return st


def kvq_decode_attention_paged(cfg, cache, layer, block_table, num_blocks, tokens, seq_tokens, q,
                               out, workspace, workspace_bytes=None, k_scale=None, v_scale=None,
                               stream=None, check=True):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().kvq_decode_attention_paged(ctypes.byref(cfg), _ptr(cache), layer, _ptr(block_table),
                                          block_table.shape[1], num_blocks, tokens,
                                          _ptr(seq_tokens), _ptr(q), _ptr(k_scale), _ptr(v_scale),
                                          _ptr(out), _ptr(workspace), workspace_bytes,
                                          _stream(stream))
    if check and st != KVQ_OK:
        raise KvqError(st, "kvq_decode_attention_paged")
    return st


# ---- allocation helpers (torch memory only) ----------------------------------

def alloc_cache(cfg, device="cuda", zero=True):
    import torch
    n = kvq_cache_bytes(cfg, cfg.max_tokens, KVQ_BYTES_CACHE)
    return (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device=device)


def alloc_workspace(cfg, tokens=None, device="cuda"):
    """Zero-filled decode workspace for calls over up to `tokens` tokens."""
    import torch
    n = kvq_cache_bytes(cfg, cfg.max_tokens if tokens is None else tokens, KVQ_BYTES_WORKSPACE)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)
