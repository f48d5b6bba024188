"""Oracle: a whole quantised KV cache, appended to and attended over
(test infrastructure only).

The oracle keeps every appended token exactly (its float32 value and the raw
bits of its input dtype) and derives the cache from that history each time it
is asked, which makes the result independent of how the appends were
chunked by construction:

* KIVI: with T tokens held, tokens [0, q(T)) are encoded in 32-token groups
  (keys per channel at `bits`, values per token at `v_bits`, which may be
  narrower: "Quantizing the KV cache", How the KV cache is quantized, names
  separate key and value cache types) and the newest T - q(T) sit in the
  residual ring unquantised, slot t mod (R + 32) ("Quantizing the KV cache":
  a window of the last R tokens is left unrounded, a full window is quantised as a
  group; KIVI How It Works: recent tokens kept in 16-bit).
* SYM_TOKEN / FP8 (E4M3FN or E5M2): every token is encoded as it arrives ("Quantising the
  Cache.", Workshop: rounded before it enters the cache).
* BF16_CACHE: every token is stored as bfloat16 as it arrives (the 16-bit
  baseline of "Quantizing the KV cache", "The other big memory user").
* FP8K_SYMV: keys and values in different cache types ("Quantizing the KV
  cache", How the KV cache is quantized: separate key and value cache
  types): each token's key encoded as FP8 E4M3 with the KV head's static key
  scale and its value symmetric per token at v_bits, as it arrives.
* FP8K_KIVIV: as FP8K_SYMV with each token's value encoded by KIVI's
  per-token Q_b at v_bits (KIVI How It Works: values per token), as it
  arrives (values need no group of later tokens, so no residual ring).

Decode attention (``decode``) dequantises in float64, applies the rotary
embedding to keys at their positions and to the query at position T-1 when
rope_theta > 0 (KVQuant Summary: keys cached before RoPE), and takes the
float64 softmax-weighted sum of value rows ("Quantizing the KV cache", "Why
values per token"). A ragged batch (per-sequence token counts, the serving
case of the KIVI page's Key points, where KIVI pairs with PagedAttention)
attends each sequence to its own first T_b tokens, query at T_b - 1.
"""

import numpy as np

from . import accounting, attention, codec, layout, rope

KIVI, SYM_TOKEN, FP8_E4M3, BF16_CACHE, FP8_E5M2, FP8K_SYMV, FP8K_KIVIV = (
    accounting.KIVI, accounting.SYM_TOKEN, accounting.FP8_E4M3, accounting.BF16_CACHE,
    accounting.FP8_E5M2, accounting.FP8K_SYMV, accounting.FP8K_KIVIV)
PAGE = 32


def bf16_bits_to_f32(raw):
    """bfloat16 bit patterns (uint16) to their exact float32 values."""
    raw = np.asarray(raw, np.uint16)
    return (raw.astype(np.uint32) << 16).view(np.float32)


class OracleCache:
    """in_dtype is "f32" (inputs float32) or "bf16" (inputs uint16 bit patterns)."""

    def __init__(self, scheme, bits, layers, batch, kv_heads, head_dim, capacity,
                 residual=0, in_dtype="bf16", v_bits=None, outliers=0):
        if scheme in (FP8K_SYMV, FP8K_KIVIV):
            v_bits = 8 if v_bits is None else v_bits   # the value codes' width when not given
            assert residual == 0 and bits == 8 and v_bits in (2, 3, 4, 8) and not outliers
        elif scheme != KIVI:
            assert residual == 0 and v_bits in (None, bits) and not outliers
        self.outliers = outliers          # KIVI: dense-and-sparse with one outlier per vector
        self.scheme, self.bits, self.layers, self.batch = scheme, bits, layers, batch
        self.v_bits = bits if v_bits is None else v_bits   # KIVI value codes
        self.kv_heads, self.d, self.capacity = kv_heads, head_dim, capacity
        self.residual, self.in_dtype = residual, in_dtype
        self.itemsize = 2 if in_dtype == "bf16" else 4
        self.raw_k = [None] * layers      # [B, T, Hkv, d] raw input (uint16 or float32)
        self.raw_v = [None] * layers
        self.k_scale = [None] * layers    # FP8: float32 [Hkv] per layer
        self.v_scale = [None] * layers

    # ---- appends ----------------------------------------------------------
    def tokens(self, layer):
        return 0 if self.raw_k[layer] is None else self.raw_k[layer].shape[1]

    def append(self, layer, k_new, v_new, k_scale=None, v_scale=None):
        k_new, v_new = np.asarray(k_new), np.asarray(v_new)
        assert k_new.shape == v_new.shape and k_new.shape[0] == self.batch
        assert self.tokens(layer) + k_new.shape[1] <= self.capacity
        if self.scheme in (FP8K_SYMV, FP8K_KIVIV):   # a static key scale only
            ks = np.asarray(k_scale, np.float32)
            if self.k_scale[layer] is not None:
                assert np.array_equal(ks, self.k_scale[layer])
            self.k_scale[layer] = ks
        if self.scheme in (FP8_E4M3, FP8_E5M2):
            ks = np.asarray(k_scale, np.float32)
            vs = np.asarray(v_scale, np.float32)
            if self.k_scale[layer] is not None:   # static per-head scales
                assert np.array_equal(ks, self.k_scale[layer])
                assert np.array_equal(vs, self.v_scale[layer])
            self.k_scale[layer], self.v_scale[layer] = ks, vs
        if self.raw_k[layer] is None:
            self.raw_k[layer], self.raw_v[layer] = k_new.copy(), v_new.copy()
        else:
            self.raw_k[layer] = np.concatenate([self.raw_k[layer], k_new], axis=1)
            self.raw_v[layer] = np.concatenate([self.raw_v[layer], v_new], axis=1)

    def values(self, layer):
        """Exact float32 values of all held tokens, [B, T, Hkv, d] each."""
        if self.in_dtype == "bf16":
            return bf16_bits_to_f32(self.raw_k[layer]), bf16_bits_to_f32(self.raw_v[layer])
        return (np.asarray(self.raw_k[layer], np.float32),
                np.asarray(self.raw_v[layer], np.float32))

    def fp8_format(self):
        return "e5m2" if self.scheme == FP8_E5M2 else "e4m3"

    # ---- byte image -------------------------------------------------------
    def slab_size(self):
        return accounting.slab_bytes(self.scheme, self.d, self.bits, self.capacity,
                                     self.residual, self.itemsize, self.v_bits, self.outliers)

    def page_size(self):
        return accounting.page_bytes(self.scheme, self.d, self.bits, self.v_bits, self.outliers)

    def slab_image(self, layer, b, h):
        """(bytes, mask) of one slab for the tokens held now."""
        size = self.slab_size()
        buf = np.zeros(size, np.uint8)
        mask = np.zeros(size, np.uint8)
        T = self.tokens(layer)
        if T == 0:
            return buf, mask
        K, V = self.values(layer)
        K, V = K[b, :, h, :], V[b, :, h, :]
        ps = self.page_size()
        if self.scheme == KIVI:
            q, _ = accounting.flush_plan(T, self.residual)
            for p in range(q // PAGE):
                pb, pm = layout.kivi_page(K[p * PAGE:(p + 1) * PAGE], V[p * PAGE:(p + 1) * PAGE],
                                          self.bits, self.v_bits, self.outliers)
                buf[p * ps:(p + 1) * ps], mask[p * ps:(p + 1) * ps] = pb, pm
            n_pages = accounting.pages_per_slab(KIVI, self.capacity, self.residual)
            ring0 = n_pages * ps
            slots = self.residual + PAGE
            row = self.d * self.itemsize
            rk = np.ascontiguousarray(self.raw_k[layer][b, :, h, :]).view(np.uint8).reshape(T, row)
            rv = np.ascontiguousarray(self.raw_v[layer][b, :, h, :]).view(np.uint8).reshape(T, row)
            for t in range(q, T):
                s = t % slots
                ko = ring0 + s * row
                vo = ring0 + (slots + s) * row
                buf[ko:ko + row], mask[ko:ko + row] = rk[t], 0xFF
                buf[vo:vo + row], mask[vo:vo + row] = rv[t], 0xFF
        else:
            for p in range(-(-T // PAGE)):
                n = min(PAGE, T - p * PAGE)
                k32 = np.zeros((PAGE, self.d), np.float32)
                v32 = np.zeros((PAGE, self.d), np.float32)
                k32[:n], v32[:n] = K[p * PAGE:p * PAGE + n], V[p * PAGE:p * PAGE + n]
                if self.scheme == SYM_TOKEN:
                    pb, pm = layout.sym_page(k32, v32, self.bits, n)
                elif self.scheme == BF16_CACHE:
                    pb, pm = layout.bf16_page(k32, v32, n)
                elif self.scheme == FP8K_SYMV:
                    pb, pm = layout.fp8k_symv_page(k32, v32, self.k_scale[layer][h], self.v_bits, n)
                elif self.scheme == FP8K_KIVIV:
                    pb, pm = layout.fp8k_kiviv_page(k32, v32, self.k_scale[layer][h], self.v_bits, n)
                else:
                    pb, pm = layout.fp8_page(k32, v32, self.k_scale[layer][h],
                                             self.v_scale[layer][h], n, self.fp8_format())
                buf[p * ps:(p + 1) * ps], mask[p * ps:(p + 1) * ps] = pb, pm
        return buf, mask

    def cache_image(self):
        """(bytes, mask) of the whole cache, slabs ordered (layer, seq, KV head)."""
        bufs, masks = [], []
        for layer in range(self.layers):
            for b in range(self.batch):
                for h in range(self.kv_heads):
                    bb, mm = self.slab_image(layer, b, h)
                    bufs.append(bb)
                    masks.append(mm)
        return np.concatenate(bufs), np.concatenate(masks)

    # ---- dequantised cache and attention -----------------------------------
    def dequantized(self, layer):
        """K^, V^ as float64 [B, Hkv, T, d] (no rotary embedding)."""
        K, V = self.values(layer)
        B, T, H, d = K.shape
        K = np.transpose(K, (0, 2, 1, 3))        # [B, H, T, d]
        V = np.transpose(V, (0, 2, 1, 3))
        kh = np.empty((B, H, T, d))
        vh = np.empty((B, H, T, d))
        if self.scheme == KIVI:
            q, _ = accounting.flush_plan(T, self.residual)
            for p in range(q // PAGE):
                sl = slice(p * PAGE, (p + 1) * PAGE)
                if self.outliers:
                    kh[:, :, sl] = codec.kivi_dequantize_sparse(
                        *codec.kivi_quantize_sparse(K[:, :, sl], self.bits, axis=2), axis=2)
                    vh[:, :, sl] = codec.kivi_dequantize_sparse(
                        *codec.kivi_quantize_sparse(V[:, :, sl], self.v_bits, axis=3), axis=3)
                    continue
                kc, ks, kz = codec.kivi_quantize(K[:, :, sl], self.bits, axis=2)
                vc, vs, vz = codec.kivi_quantize(V[:, :, sl], self.v_bits, axis=3)
                kh[:, :, sl] = codec.kivi_dequantize(kc, ks, kz, axis=2)
                vh[:, :, sl] = codec.kivi_dequantize(vc, vs, vz, axis=3)
            kh[:, :, q:] = K[:, :, q:]
            vh[:, :, q:] = V[:, :, q:]
        elif self.scheme == BF16_CACHE:
            kh[:] = codec.bf16_decode(codec.bf16_encode(K))
            vh[:] = codec.bf16_decode(codec.bf16_encode(V))
        elif self.scheme in (FP8K_SYMV, FP8K_KIVIV):
            ksc = self.k_scale[layer][None, :, None, None]
            kh[:] = codec.fp8_dequantize(codec.fp8_quantize(K, ksc, "e4m3"), ksc, "e4m3")
            if self.scheme == FP8K_SYMV:
                vc, vs = codec.sym_quantize(V, self.v_bits, axis=3)
                vh[:] = codec.sym_dequantize(vc, vs, axis=3)
            else:
                vc, vs, vz = codec.kivi_quantize(V, self.v_bits, axis=3)
                vh[:] = codec.kivi_dequantize(vc, vs, vz, axis=3)
        elif self.scheme == SYM_TOKEN:
            kc, ks = codec.sym_quantize(K, self.bits, axis=3)
            vc, vs = codec.sym_quantize(V, self.bits, axis=3)
            kh[:] = codec.sym_dequantize(kc, ks, axis=3)
            vh[:] = codec.sym_dequantize(vc, vs, axis=3)
        else:
            ksc = self.k_scale[layer][None, :, None, None]
            vsc = self.v_scale[layer][None, :, None, None]
            f = self.fp8_format()
            kh[:] = codec.fp8_dequantize(codec.fp8_quantize(K, ksc, f), ksc, f)
            vh[:] = codec.fp8_dequantize(codec.fp8_quantize(V, vsc, f), vsc, f)
        return kh, vh

    def decode(self, layer, q, sm_scale=None, rope_theta=0.0, seq_tokens=None):
        """Attention of q [B, Hq, d] (float values) over the held tokens.

        seq_tokens (optional, one count per sequence, 1 <= T_b <= T): a ragged
        batch, where sequence b attends to its first T_b tokens only and its
        query sits at position T_b - 1. The cache itself stays as held (for
        KIVI its page/ring split follows T, the fill level), so the tokens a
        sequence reads are exactly those rows of the dequantised cache."""
        kh, vh = self.dequantized(layer)
        q = np.asarray(q, np.float64)
        B, T = kh.shape[0], kh.shape[2]
        if sm_scale is None or sm_scale == 0:
            sm_scale = 1.0 / np.sqrt(self.d)
        lens = [T] * B if seq_tokens is None else [int(x) for x in seq_tokens]
        out = np.zeros(q.shape)
        for b in range(B):
            Tb = lens[b]
            assert 1 <= Tb <= T, (b, Tb, T)
            kb, vb, qb = kh[b:b + 1, :, :Tb], vh[b:b + 1, :, :Tb], q[b:b + 1]
            if rope_theta > 0:
                kb = rope.rotate(kb, np.arange(Tb), rope_theta)
                qb = rope.rotate(qb, np.full(qb.shape[:-1], Tb - 1), rope_theta)
            out[b] = attention.decode(qb, kb, vb, sm_scale)[0]
        return out


    def decode_multi(self, layer, q, sm_scale=None, rope_theta=0.0):
        """Several new queries per sequence (q [B, n_q, Hq, d]): the cache holds
        T tokens whose last n_q are the queries' own tokens, and query i, at
        position T - n_q + i, attends causally to tokens [0, T - n_q + i] --
        the masked-prefix decode with T_b = T - n_q + i + 1 (the same cache,
        several more queries per step: chunked prefill or speculative
        verification over the quantised cache)."""
        q = np.asarray(q, np.float64)
        B, nq = q.shape[:2]
        T = self.tokens(layer)
        out = np.zeros(q.shape)
        for i in range(nq):
            out[:, i] = self.decode(layer, q[:, i], sm_scale, rope_theta,
                                    seq_tokens=[T - nq + i + 1] * B)
        return out

class RaggedCache:
    """A batch whose sequences hold different numbers of tokens (a ragged
    batch: the serving case of the KIVI page's Key points, where KIVI pairs
    with PagedAttention): one single-sequence OracleCache per sequence, each
    with its own fill level T_b -- and so, for KIVI, its own split of tokens
    between quantised pages [0, q(T_b)) and the ring [q(T_b), T_b). The byte
    image is the slabs of the per-sequence caches in (layer, sequence, KV head)
    order; decode attends each sequence to its own T_b tokens, its query at
    T_b - 1 (test infrastructure only)."""

    def __init__(self, scheme, bits, layers, batch, kv_heads, head_dim, capacity, residual=0,
                 in_dtype="bf16", v_bits=None, outliers=0):
        self.layers, self.batch, self.kv_heads = layers, batch, kv_heads
        self.seqs = [OracleCache(scheme, bits, layers, 1, kv_heads, head_dim, capacity,
                                 residual=residual, in_dtype=in_dtype, v_bits=v_bits,
                                 outliers=outliers)
                     for _ in range(batch)]

    def tokens(self, layer):
        return [c.tokens(layer) for c in self.seqs]

    def append(self, layer, b, k_new, v_new, k_scale=None, v_scale=None):
        """Appends k_new, v_new [n, Hkv, d] (raw input values) to sequence b;
        n = 0 leaves it unchanged."""
        k_new, v_new = np.asarray(k_new), np.asarray(v_new)
        if k_new.shape[0] == 0:
            return
        self.seqs[b].append(layer, k_new[None], v_new[None], k_scale, v_scale)

    def cache_image(self):
        """(bytes, mask) of the whole cache, slabs ordered (layer, seq, KV head)."""
        bufs, masks = [], []
        for layer in range(self.layers):
            for b in range(self.batch):
                for h in range(self.kv_heads):
                    bb, mm = self.seqs[b].slab_image(layer, 0, h)
                    bufs.append(bb)
                    masks.append(mm)
        return np.concatenate(bufs), np.concatenate(masks)

    def decode(self, layer, q, sm_scale=None, rope_theta=0.0):
        """q [B, Hq, d]: sequence b over its own T_b tokens."""
        q = np.asarray(q, np.float64)
        out = np.zeros(q.shape)
        for b in range(self.batch):
            out[b] = self.seqs[b].decode(layer, q[b:b + 1], sm_scale, rope_theta)[0]
        return out


def paged_image(cache, table, num_blocks):
    """(bytes, mask) of a paged cache (the KIVI page's Key points: KIVI pairs
    with PagedAttention, which places a sequence's pages in blocks of a shared
    pool through a block table). `cache` is an OracleCache or RaggedCache and
    `table` an int array [batch, max_blocks]: page p of sequence b (of every
    layer) sits in block table[b][p]. Buffer: the residual rings of every
    (layer, sequence, KV head) in that order, padded to 256 bytes, then per
    layer num_blocks blocks of one page per KV head. Each page and ring holds
    exactly the bytes of its slab-layout counterpart."""
    table = np.asarray(table)
    seqs = cache.seqs if isinstance(cache, RaggedCache) else None
    one = seqs[0] if seqs else cache
    layers, batch, H = one.layers, table.shape[0], one.kv_heads
    ps = one.page_size()
    P = accounting.pages_per_slab(one.scheme, one.capacity, one.residual)
    rb = accounting.ring_bytes(one.scheme, one.d, one.residual, one.itemsize)
    assert table.shape[1] >= P
    ring_region = -(-(layers * batch * H * rb) // 256) * 256
    size = ring_region + layers * num_blocks * H * ps
    buf = np.zeros(size, np.uint8)
    mask = np.zeros(size, np.uint8)
    for layer in range(layers):
        for b in range(batch):
            for h in range(H):
                sb, sm = (seqs[b].slab_image(layer, 0, h) if seqs else cache.slab_image(layer, b, h))
                for pg in range(P):
                    o = ring_region + ((layer * num_blocks + int(table[b, pg])) * H + h) * ps
                    buf[o:o + ps] = sb[pg * ps:(pg + 1) * ps]
                    mask[o:o + ps] = sm[pg * ps:(pg + 1) * ps]
                if rb:
                    o = ((layer * batch + b) * H + h) * rb
                    buf[o:o + rb] = sb[P * ps:P * ps + rb]
                    mask[o:o + rb] = sm[P * ps:P * ps + rb]
    return buf, mask
