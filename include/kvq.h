/*
 * kvq.h -- C ABI of the quantised KV-cache library (MI355X / gfx950).
 *
 * Two computations make up the hot path:
 *   (a) quantize-append: new keys/values of every sequence are encoded into a
 *       packed cache (KIVI-style asymmetric b-bit codes with a full-precision
 *       residual window, a symmetric per-head-per-token variant, or FP8 E4M3
 *       with a per-head scale);
 *   (b) decode attention: q.K^T, softmax and P.V computed straight from the
 *       packed cache, split over the token axis and merged on the GPU.
 *
 * Sources the operations follow (web pages on KV-cache quantisation):
 *   [QC]   "Quantising the Cache." (llm.curionode.com, efficient-inference /
 *          kv-quantisation): Workshop; "Twice the users for nearly nothing";
 *          Terms (per-token, per-channel).
 *   [QKV]  "Quantizing the KV cache" (learning.iampt.xyz/quantization/kv-cache):
 *          "The other big memory user" (KV-bytes equation); "How the KV cache is
 *          quantized" (FP8 KV cache); "Keys and values are shaped differently";
 *          going deeper: "Per-channel and per-token grouping" (Q_b, s) and
 *          "Why values per token" (o = sum_t p_t V_t).
 *   [KIVI] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *          (crackai.dev/papers/kivi): "How It Works" (per-channel keys,
 *          per-token values, residual length of recent tokens kept unquantised).
 *   [KVQ]  "KVQuant: Towards 10 Million Context Length LLM Inference with KV
 *          Cache Quantization" (research.elamur.ai): Summary (keys quantised
 *          before the rotary embedding).
 *
 * Conventions shared by every entry point
 *   - All device buffers are owned by the caller. The library allocates and
 *     frees nothing and keeps no global mutable state.
 *   - Device pointers must be 16-byte aligned.
 *   - Calls are asynchronous: they validate their arguments on the host, then
 *     enqueue kernels on `stream` (a hipStream_t; NULL = the default stream)
 *     and return. Inputs must stay live until the stream has passed them.
 *   - Validation happens before anything is enqueued. On any error nothing is
 *     launched and the negative status is returned.
 *   - KVQ_ERR_DEVICE is returned when a kernel launch reports an error.
 *   - Keys, values and queries must be finite; non-finite input is outside the
 *     contract and not checked.
 *   - Accuracy of decode, against softmax attention computed exactly (fp64)
 *     over the dequantised cache: max-abs error <= 2e-3 * max(1, V*(1+S/2)/128),
 *     where V = max |dequantised value| and S = sum_c |sm_scale*q_c| * K_c with
 *     K_c the largest |key| of channel c. So the error is within 2e-3 whenever
 *     V*(1+S/2) <= 128. This is a worst-case bound from the arithmetic: scores
 *     and accumulators are fp32 (score error <= 2^-20 of the summands'
 *     magnitude), softmax weights enter the value product as bfloat16 high
 *     and remainder parts (2^-17 relative). Rounding errors of real inputs do
 *     not line up, and the measured errors are far below it (1e-6 to 3e-5 on
 *     the benchmark workloads, which lie well outside the 2e-3 range of the
 *     bound). No operand saturates: a page whose folded query
 *     q * s * sm_scale * log2(e) exceeds the f16 maximum (65504) is rescaled
 *     by a power of two inside the kernel and the scaling undone on its scores.
 *     Several queries decoded four per block (kvq_decode_attention_multi with
 *     a multiple of four queries of a KIVI cache of 16-bit inputs at GQA 4
 *     without rotary keys, head_dim <= 128) take each page's keys
 *     dequantised into f16 high and
 *     remainder parts, and q' = q * sm_scale * log2(e) likewise, each scaled
 *     below 2^15 by a power of two: a score then carries, besides the bound
 *     above, up to 2^-24 * (|q'|_1 * max(1, K/2^14) + sum_c K_c * max(1,
 *     Q/2^14)) log2 units from f16 subnormals, K the page's largest |key|
 *     and Q = max_c |q'_c| (negligible unless some channel's keys or queries
 *     are tiny beside another's that reach 2^14).
 *   - Calls on distinct streams are independent; concurrent calls that touch
 *     the same cache slab or workspace race (the caller's responsibility).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 11  /* 3: ragged-batch entry points; 4: several queries per sequence;
                               5: decode without a caller workspace; 6: sparse outliers;
                               7: paged caches (block tables);
                               8: one-token append fused with decode;
                               9: keys and values in different cache types;
                               10: FP8 values of an open page in token rows;
                               11: FP8 keys with KIVI values */

/* Exported entry points (the library is built with hidden visibility). */
#if defined(__GNUC__)
#define KVQ_API __attribute__((visibility("default")))
#else
#define KVQ_API
#endif

/* ---- status codes ------------------------------------------------------ */
#define KVQ_OK               0
#define KVQ_ERR_NULL        -1  /* a required pointer is NULL                */
#define KVQ_ERR_INVALID     -2  /* a value is out of range / inconsistent    */
#define KVQ_ERR_UNSUPPORTED -3  /* valid but not built (e.g. head_dim 96)    */
#define KVQ_ERR_CAPACITY    -4  /* past_tokens + new_tokens > max_tokens     */
#define KVQ_ERR_WORKSPACE   -5  /* workspace_bytes too small                 */
#define KVQ_ERR_DEVICE      -6  /* the HIP runtime reported a launch error   */

/* ---- schemes ------------------------------------------------------------ */
/* KVQ_KIVI: asymmetric round-to-nearest, keys per channel over groups of
 *   `group` consecutive tokens, values per token (one scale and offset per
 *   token per KV head); the newest `residual` tokens stay in the input dtype.
 *   [QKV] going deeper: "Per-channel and per-token grouping"; [KIVI] How It
 *   Works. bits in {2,4,8}.
 * KVQ_SYM_TOKEN: symmetric round-to-nearest of each head's key and value at
 *   every token, one scale per (token, KV head) for K and one for V; every
 *   token is encoded on arrival. [QC] Workshop. bits in {2,4,8}.
 * KVQ_FP8_E4M3: each element divided by a static per-(layer, KV head) fp32
 *   scale and rounded to OCP FP8 E4M3FN (nearest, ties to even mantissa,
 *   saturating at +-448). [QKV] "How the KV cache is quantized", FP8 KV cache.
 *   bits must be 8.
 * KVQ_FP8_E5M2: as KVQ_FP8_E4M3 with the other FP8 format the page names,
 *   OCP E5M2 (5 exponent bits, bias 15; nearest, ties to even mantissa,
 *   saturating at +-57344, the largest finite value). bits must be 8.
 * KVQ_BF16_CACHE: no quantisation, every value stored as bfloat16 (the
 *   16-bit cache the pages compare the quantised ones against, [QKV] "The
 *   other big memory user"); the baseline for measuring what 2/4/8-bit codes
 *   save. bits must be 16.
 * KVQ_FP8K_SYMV: keys and values in different cache types ([QKV] "How the KV
 *   cache is quantized": separate key and value cache types): keys as in
 *   KVQ_FP8_E4M3 (static per-(layer, KV head) key scale), values as in
 *   KVQ_SYM_TOKEN at v_bits (one scale per (token, KV head)); every token is
 *   encoded on arrival. bits must be 8; v_bits in {2,3,4,8} (0 means 8; 3
 *   needs head_dim >= 64).
 * KVQ_FP8K_KIVIV: as KVQ_FP8K_SYMV with the values encoded as KIVI encodes
 *   them, asymmetric per (token, KV head) over the d channels at v_bits
 *   ([KIVI] How It Works: values per token), on arrival: a value vector
 *   needs no group of later tokens, so there is no residual ring. Same bits
 *   and v_bits rules. */
#define KVQ_KIVI       0
#define KVQ_SYM_TOKEN  1
#define KVQ_FP8_E4M3   2
#define KVQ_BF16_CACHE 3
#define KVQ_FP8_E5M2   4
#define KVQ_FP8K_SYMV  5
#define KVQ_FP8K_KIVIV 6

/* ---- dtypes (K/V input + residual ring, and the query) ------------------ */
#define KVQ_F32   0
#define KVQ_BF16  1

/* ---- kvq_cache_bytes kinds --------------------------------------------- */
#define KVQ_BYTES_FORMULA    0  /* batch * 2*layers*kv_heads*head_dim*tokens*bits/8 */
#define KVQ_BYTES_CACHE      1  /* exact bytes of the layout below              */
#define KVQ_BYTES_WORKSPACE  2  /* decode workspace for a call over `tokens`    */

/* Shape and encoding of one cache. All fields by value; struct_size must be
 * sizeof(kvq_config) (ABI guard). [QKV] "The other big memory user": the cache
 * is layers x KV heads x head size x tokens x bits; several query heads share
 * one KV head (grouped-query attention). */
typedef struct kvq_config {
  uint32_t struct_size;  /* = sizeof(kvq_config)                            */
  int32_t  scheme;       /* KVQ_KIVI / KVQ_SYM_TOKEN / KVQ_FP8_E4M3 /
                            KVQ_FP8_E5M2 / KVQ_BF16_CACHE                   */
  int32_t  bits;         /* 2, 4 or 8 (8 for FP8, 16 for BF16_CACHE); for
                            KIVI the bits of the key codes (see v_bits)     */
  int32_t  layers;       /* >= 1                                            */
  int32_t  q_heads;      /* kv_heads * {1, 2, 4, 8}                        */
  int32_t  kv_heads;     /* 1..65535                                        */
  int32_t  head_dim;     /* 32, 64, 128 or 256                              */
  int32_t  batch;        /* 1..65535 sequences (of one length; of their own
                            with the _ragged entry points)                 */
  int64_t  max_tokens;   /* capacity per sequence, < 2^36                   */
  int32_t  group;        /* tokens per page / key group; must be 32         */
  int32_t  residual;     /* KIVI: R >= 0 newest tokens kept unquantised;
                            must be 0 for the other schemes                 */
  int32_t  in_dtype;     /* dtype of k_new/v_new and of the residual ring   */
  int32_t  q_dtype;      /* dtype of the decode query                       */
  double   rope_theta;   /* > 0: keys are cached before the rotary embedding
                            and decode rotates dequantised keys (position t)
                            and the query (position tokens-1) [KVQ] Summary;
                            0: no rotation                                  */
  float    sm_scale;     /* softmax scale; 0 selects 1/sqrt(head_dim)       */
  int32_t  num_splits;   /* decode token splits per (seq, KV head);
                            0 = automatic, else an upper bound              */
  int32_t  v_bits;       /* KIVI: bits of the value codes, 2, 4 or 8 and at
                            most `bits` (keys take the wider codes: a few
                            key channels carry large values, and rounding
                            costs keys more than values, [QKV] "How the KV
                            cache is quantized", INT8 / INT4 blocks with
                            separate key and value cache types); 0 = `bits`.
                            FP8K_SYMV / FP8K_KIVIV: bits of the value
                            codes, 2, 3, 4 or 8 (0 = 8). Other schemes: 0 or
                            equal to `bits`.                               */
  int32_t  outliers;     /* KIVI: 1 = dense-and-sparse pages (each key
                            channel's 32 tokens and each value token keep
                            their largest-magnitude value exactly in a side
                            matrix, [KVQ] Summary: a small fraction of
                            outliers moved, per vector, into a separate
                            sparse representation); 0 = dense pages. Must
                            be 0 for the other schemes.                    */
} kvq_config;

/* ==== Cache layout, version 1 =============================================
 * The cache is one byte buffer. It holds, in this order, one slab per
 * (layer, sequence, KV head):   slab_index = (layer*batch + seq)*kv_heads + h.
 * A slab is `P` pages followed (KIVI only) by the residual ring. Every page
 * holds `group` = 32 consecutive tokens of one (layer, seq, KV head); page p
 * covers tokens [32p, 32p+32).
 *
 * Packing: b-bit field i of a packed run occupies bits [i*b, (i+1)*b) of the
 * run read as a little-endian bit stream (LSB of byte 0 first).
 * "K rows": the page's 32 tokens one after another, each token's d channel
 *           codes contiguous (field index = channel).
 * "V cols": the page's d channels one after another, each channel's 32 token
 *           codes contiguous (field index = token).
 * d = head_dim, b = bits; KIVI keys take bk = bits and values bv = v_bits (or
 * bits when v_bits is 0). All sizes below are multiples of 16 bytes and every
 * page size is a multiple of 256 bytes.
 *
 * KIVI page (4*d*(bk+bv) + 8*d + 256 bytes; 8*d*b + 8*d + 256 when bk = bv
 * = b), P = floor(max(0, max_tokens-R)/32):
 *   Kc  K rows, unsigned bk-bit codes     32*d*bk/8 bytes
 *   Ks  fp32 scale per channel            4*d
 *   Kz  fp32 offset (group min)           4*d
 *   Vc  V cols, unsigned bv-bit codes     32*d*bv/8
 *   Vs  fp32 scale per token       128
 *   Vz  fp32 offset per token      128
 *   With outliers = 1 the page continues with its side matrix
 *   (5*d + 160 bytes, padded to a multiple of 256; the padding is unspecified):
 *   Ko  fp32 key outlier per channel, the exact input value   4*d
 *   Vo  fp32 value outlier per token, the exact input value   128
 *   Ki  uint8 token (0..31) of each channel's key outlier     d
 *   Vi  uint8 channel (0..d-1) of each token's value outlier  32
 *   Ring after the P pages: (R+32) K rows then (R+32) V rows, each d values of
 *   in_dtype; token t lives in slot t mod (R+32) while it is unquantised.
 * SYM_TOKEN page (8*d*b + 256 bytes), P = ceil(max_tokens/32):
 *   Kc  K rows, b-bit two's-complement codes   32*d*b/8
 *   Ks  fp32 scale per token                   128
 *   Vc  V cols, b-bit two's-complement codes   32*d*b/8
 *   Vs  fp32 scale per token                   128
 * FP8_E4M3 / FP8_E5M2 page (64*d bytes), P = ceil(max_tokens/32):
 *   Kc  K rows, one FP8 byte per value         32*d
 *   Vc  V cols, one FP8 byte per value         32*d
 *   except the cache's open page: while the last page of a sequence holds
 *   fewer than 32 tokens its Vc region holds V rows (token r's d codes at
 *   r*d), so that appending a token writes one contiguous row; the append
 *   that fills the page rewrites the region as V cols.
 * BF16_CACHE page (128*d bytes), P = ceil(max_tokens/32):
 *   Kc  K rows, bfloat16 per value (16-bit fields)   64*d
 *   Vc  V cols, bfloat16 per value                   64*d
 * FP8K_SYMV page (32*d + 4*d*bv + 256 bytes), P = ceil(max_tokens/32):
 *   Kc  K rows, one FP8 E4M3 byte per value            32*d
 *   Vc  V cols, bv-bit two's-complement codes          32*d*bv/8
 *   Vs  fp32 scale per token                           128
 *   (then 128 bytes of padding, unspecified)
 * FP8K_KIVIV page (32*d + 4*d*bv + 256 bytes), P = ceil(max_tokens/32):
 *   Kc  K rows, one FP8 E4M3 byte per value            32*d
 *   Vc  V cols, unsigned bv-bit codes                  32*d*bv/8
 *   Vs  fp32 scale per token                           128
 *   Vz  fp32 offset (minimum) per token                128
 *
 * Which tokens are quantised (KIVI), for a cache holding T tokens:
 *   q(T) = 32*floor(max(0, T-R)/32) tokens live in pages [0, q(T)/32); the
 *   other n_r = T - q(T) tokens live in the ring. So a window of at least the
 *   last R tokens stays unquantised, and whenever R+32 tokens are unquantised
 *   the oldest 32 are encoded as one group. [QKV] "Keys and values are shaped
 *   differently" (window of recent tokens quantised as a group once it fills)
 *   and going deeper (a full-precision window of recent tokens); [KIVI] How
 *   It Works (residual length).
 * Encoding of one KIVI group (fp32 arithmetic, IEEE division, ties-to-even
 * rounding, no fused multiply-add), L = 2^bk - 1 for keys and 2^bv - 1 for
 * values, per key channel over the 32 tokens of the page and per value token
 * over its d channels:
 *   mn = min x (+0 replaces -0), mx = max x, s = (mx - mn) / L,
 *   code = s == 0 ? 0 : clamp(rint((x - mn) / s), 0, L),  stored offset = mn;
 *   dequantised value = code*s + mn.  [QKV] going deeper, Q_b and s.
 *   FP8K_KIVIV values are encoded the same way, per value token on arrival.
 * Dense-and-sparse KIVI group (outliers = 1): the value of largest magnitude
 *   |x| of each vector (lowest index among equal magnitudes) goes to the side
 *   matrix with its index; mn, mx and s above are taken over the other values
 *   of the vector, and the moved position holds code 0. Dequantised: the
 *   side matrix's value at that position, code*s + mn elsewhere. [KVQ]
 *   Summary (outliers per vector in a sparse representation).
 * SYM_TOKEN, per (token, KV head), K and V separately, Q = 2^(b-1) - 1:
 *   s = max|x| / Q, code = s == 0 ? 0 : clamp(rint(x / s), -Q, Q);
 *   dequantised value = code*s.  [QC] Workshop.
 * FP8_E4M3: code = E4M3FN(x / scale[h]) (round to nearest, ties to even
 *   mantissa, |y| >= 448 -> +-448, sign kept); dequantised = value*scale[h].
 * FP8_E5M2: code = E5M2(x / scale[h]) (round to nearest, ties to even
 *   mantissa, |y| >= 57344 -> +-57344, sign kept); dequantised = value*scale[h].
 * BF16_CACHE: bf16 input is stored bit for bit; fp32 input is rounded to
 *   bfloat16 (nearest, ties to even); the stored value is used as is.
 * ========================================================================== */

/* Bytes for `tokens` tokens per sequence. Host-only; never touches a device.
 *   KVQ_BYTES_FORMULA:   batch * 2*layers*kv_heads*head_dim*tokens*bits/8, the
 *                        KV-bytes equation of [QKV] "The other big memory
 *                        user" with scales ignored (as in [QC] Workshop);
 *                        with KIVI value codes of v_bits, the keys' and the
 *                        values' halves are counted at their own widths:
 *                        batch*layers*kv_heads*head_dim*tokens*(bits+v_bits)/8.
 *   KVQ_BYTES_CACHE:     exact size of the layout above for capacity `tokens`
 *                        (all layers, all sequences).
 *   KVQ_BYTES_WORKSPACE: decode workspace needed by a call over `tokens`
 *                        cached tokens (monotone in `tokens`).
 * Returns the byte count (>= 0) or a negative status. */
KVQ_API int64_t kvq_cache_bytes(const kvq_config* cfg, int64_t tokens, int32_t kind);

/* Quantize-append: append `new_tokens` tokens to every sequence of `layer`.
 *   cache        device, >= kvq_cache_bytes(cfg, max_tokens, KVQ_BYTES_CACHE)
 *   past_tokens  tokens already held per sequence (all sequences equal)
 *   k_new, v_new device [batch][new_tokens][kv_heads][head_dim], in_dtype
 *   k_scale,
 *   v_scale      FP8 (either format) only: device fp32 [kv_heads], this layer's per-head
 *                scales (must be > 0); FP8K_SYMV / FP8K_KIVIV: k_scale
 *                only (v_scale ignored); NULL for the other schemes
 * Requires past_tokens + new_tokens <= max_tokens (else KVQ_ERR_CAPACITY).
 * new_tokens == 0 is a no-op. Appending in any chunking (one call of T tokens
 * or T calls of one token) leaves identical bytes in every defined field.
 * Steps [QKV] going deeper; [KIVI] How It Works; [QC] Workshop; [QKV] FP8. */
KVQ_API int32_t kvq_quantize_append(const kvq_config* cfg, void* cache, int32_t layer,
                            int64_t past_tokens, int64_t new_tokens,
                            const void* k_new, const void* v_new,
                            const float* k_scale, const float* v_scale,
                            void* stream);

/* Quantize-append for a ragged batch: sequence b appends seq_new[b] tokens
 * (rows 0 .. seq_new[b]-1 of its slice of k_new / v_new) after the
 * seq_past[b] tokens it holds, each sequence keeping its own fill level (and,
 * for KIVI, its own split between quantised pages and the ring). Serving
 * batches hold requests of different lengths: [KIVI] Key points (KIVI pairs
 * with PagedAttention for production serving).
 *   seq_past,
 *   seq_new   device int64 [batch] (8-byte aligned), read by the kernels; the
 *             host cannot check them, so each sequence's counts are clamped on
 *             the device to 0 <= past <= max_tokens and
 *             0 <= new <= min(new_max, max_tokens - past)
 *   new_max   rows per sequence in k_new / v_new (>= every seq_new[b]);
 *             new_max == 0 is a no-op; new_max > max_tokens is KVQ_ERR_CAPACITY
 *   k_new,
 *   v_new     device [batch][new_max][kv_heads][head_dim], in_dtype
 * Other arguments and errors as kvq_quantize_append. A call with every
 * seq_past[b] = past and seq_new[b] = new_max writes the same bytes as
 * kvq_quantize_append(past, new_max). */
KVQ_API int32_t kvq_quantize_append_ragged(const kvq_config* cfg, void* cache, int32_t layer,
                                   const int64_t* seq_past, const int64_t* seq_new,
                                   int64_t new_max, const void* k_new, const void* v_new,
                                   const float* k_scale, const float* v_scale,
                                   void* stream);

/* Decode attention over the `tokens` cached tokens of `layer`:
 *   out[b][h][:] = sum_t p_t * V^[t],  p = softmax_t(sm_scale * q[b][h].K^[t])
 * where K^, V^ are the dequantised cache and query head h reads KV head
 * floor(h / (q_heads/kv_heads)).  [QKV] going deeper, "Why values per token".
 * With rope_theta > 0 the dequantised key at position t and the query (at
 * position tokens-1) are rotated by the rotary embedding: channel pairs
 * (2i, 2i+1) turned by angle pos * theta^(-2i/head_dim).  [KVQ] Summary.
 *   q          device [batch][q_heads][head_dim], q_dtype
 *   k_scale,
 *   v_scale    FP8 only: as for append (FP8K_SYMV / FP8K_KIVIV: k_scale
 *              only, v_scale ignored); NULL otherwise
 *   out        device fp32 [batch][q_heads][head_dim]
 *   workspace  device, >= kvq_cache_bytes(cfg, tokens, KVQ_BYTES_WORKSPACE);
 *              zero-filled before its first use. It begins with one int32
 *              arrival counter per (sequence, KV head), followed by the split
 *              partials; every call leaves all of it at zero again (a partial
 *              slot holds the complement of a float's bits, so it reads zero
 *              until its block has written it in the call). A workspace may
 *              be shared by calls that run one after another (any layer,
 *              config or token count it is large enough for), never by calls
 *              that may overlap
 * Requires 1 <= tokens <= max_tokens and that the cache holds `tokens` tokens.
 */
KVQ_API int32_t kvq_decode_attention(const kvq_config* cfg, const void* cache,
                             int32_t layer, int64_t tokens, const void* q,
                             const float* k_scale, const float* v_scale,
                             float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* One decode step of every sequence: kvq_quantize_append(cfg, cache, layer,
 * past_tokens, 1, k_new, v_new, ...) followed by kvq_decode_attention over
 * past_tokens + 1 tokens -- the same cache bytes and the same output, bit for
 * bit. Generation appends the token whose query attends next ([QKV] going
 * deeper; [KIVI] How It Works: each new token enters the full-precision
 * window). When the new token lands in the residual window of a KIVI cache
 * that decodes on the matrix-core kernel (no page to encode on this step),
 * both happen in one launch: the decode reads the new rows from k_new/v_new
 * and stores them into their ring slot. Otherwise (a page flush, other
 * schemes) the append's kernels run first.
 *   past_tokens  tokens held before the call; past_tokens < max_tokens
 *   k_new, v_new device [batch][1][kv_heads][head_dim], in_dtype
 *   q, out, workspace, k_scale, v_scale: as kvq_decode_attention over
 *                past_tokens + 1 tokens
 * Errors: those of both calls, checked before anything is launched. */
KVQ_API int32_t kvq_append_decode(const kvq_config* cfg, void* cache, int32_t layer,
                          int64_t past_tokens, const void* k_new, const void* v_new,
                          const float* k_scale, const float* v_scale, const void* q,
                          float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention over a ragged batch: sequence b holds seq_tokens[b]
 * tokens (its own fill level, as appended by kvq_quantize_append_ragged; for
 * KIVI its quantised pages are [0, q(seq_tokens[b])) and the rest sits in its
 * ring) and attends to all of them, its query at position seq_tokens[b] - 1
 * (for the rotary embedding). seq_tokens[b] must be what the sequence holds:
 * a smaller count is not a prefix of it (KIVI's page/ring split and the
 * layout of an FP8 cache's open last page follow the fill level).
 * Everything else is as kvq_decode_attention.
 * Serving batches hold requests of different lengths: [KIVI] Key points
 * (KIVI pairs with PagedAttention for production serving).
 *   tokens      bound on every seq_tokens[b] (<= max_tokens); the split plan
 *               and the workspace size follow it
 *   seq_tokens  device int64 [batch] (8-byte aligned), read by the kernels;
 *               each value is clamped to [1, tokens] on the device (the host
 *               cannot check it)
 *   workspace   as for kvq_decode_attention over `tokens` (same size)
 * Other arguments, requirements and errors as kvq_decode_attention;
 * seq_tokens == NULL is KVQ_ERR_NULL. With every seq_tokens[b] = tokens the
 * result is kvq_decode_attention's, bit for bit. */
KVQ_API int32_t kvq_decode_attention_ragged(const kvq_config* cfg, const void* cache,
                                    int32_t layer, int64_t tokens,
                                    const int64_t* seq_tokens, const void* q,
                                    const float* k_scale, const float* v_scale,
                                    float* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ==== Paged cache (block table) ============================================
 * KIVI reduces the bytes per token and paged allocation removes the slab
 * fragmentation; serving needs both ([KIVI] Key points: KIVI pairs with
 * PagedAttention). A paged cache is one byte buffer holding, in this order:
 *   rings   one residual ring per (layer, sequence, KV head), index
 *           (layer*batch + seq)*kv_heads + h, each 2*(R+32)*d*in_bytes bytes
 *           as in layout v1 (KIVI only; empty for the other schemes); the
 *           region is padded to a multiple of 256 bytes;
 *   blocks  per layer, num_blocks physical blocks; block n of layer l holds
 *           one page (layout v1, page_bytes) per KV head: page of head h at
 *           blocks + ((l*num_blocks + n)*kv_heads + h)*page_bytes.
 * block_table: device int32 [batch][max_blocks]; entry [b][p] is the block
 * that holds page p (tokens 32p..32p+31) of sequence b in every layer. A
 * sequence may use any blocks; two sequences must not share a block (the
 * caller's allocator owns the table). Entries outside [0, num_blocks) are
 * clamped into it on the device (every access stays inside the buffer; the
 * result is then meaningless, not a fault). max_blocks must cover a full
 * sequence: max_blocks >= floor(max(0, max_tokens - R)/32) pages for KIVI,
 * ceil(max_tokens/32) for the other schemes (else KVQ_ERR_CAPACITY).
 * The paged calls take per-sequence counts as the ragged ones do. With the
 * same counts, every page holds the same bytes as in the slab layout, and
 * decode gives the same result bit for bit.
 * ========================================================================== */

/* Bytes of a paged cache with num_blocks blocks per layer (rings included),
 * or a negative status. Host-only. */
KVQ_API int64_t kvq_paged_cache_bytes(const kvq_config* cfg, int64_t num_blocks);

/* kvq_quantize_append_ragged into a paged cache: sequence b's page p is
 * written in block block_table[b][p] (KIVI rings in the ring region).
 *   block_table  device int32 [batch][max_blocks], 4-byte aligned
 *   max_blocks   row length of the table (see above)
 *   num_blocks   blocks per layer in `cache` (1 .. 2^31-1); `cache` holds at
 *                least kvq_paged_cache_bytes(cfg, num_blocks) bytes
 * Other arguments, clamping of the counts, and errors as
 * kvq_quantize_append_ragged; a NULL table is KVQ_ERR_NULL. */
KVQ_API int32_t kvq_quantize_append_paged(const kvq_config* cfg, void* cache, int32_t layer,
                                  const int32_t* block_table, int32_t max_blocks,
                                  int64_t num_blocks, const int64_t* seq_past,
                                  const int64_t* seq_new, int64_t new_max, const void* k_new,
                                  const void* v_new, const float* k_scale, const float* v_scale,
                                  void* stream);

/* kvq_decode_attention_ragged over a paged cache (block table as for
 * kvq_quantize_append_paged). Workspace, arguments and errors as
 * kvq_decode_attention_ragged. */
KVQ_API int32_t kvq_decode_attention_paged(const kvq_config* cfg, const void* cache,
                                   int32_t layer, const int32_t* block_table,
                                   int32_t max_blocks, int64_t num_blocks, int64_t tokens,
                                   const int64_t* seq_tokens, const void* q,
                                   const float* k_scale, const float* v_scale, float* out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Decode attention for several new queries per sequence, causally (chunked
 * prefill, or verifying speculated tokens, over the quantised cache): the
 * cache holds `tokens` tokens per sequence, the last n_queries of which are
 * the queries' own tokens, and query i (position tokens - n_queries + i)
 * attends to tokens [0, tokens - n_queries + i]: the same softmax as
 * kvq_decode_attention over that prefix, with the KIVI page/ring split of
 * the whole cache ([QKV] going deeper, "Why values per token"; one query per
 * row as kvq_decode_attention computes it).
 * Causality is over positions, not over the encoding: a KIVI cache is read
 * as it stands after all `tokens` were appended. A key page's per-channel
 * scale and offset come from all 32 of its tokens, so a query whose token
 * sits inside a quantised page reads that page's earlier keys through
 * statistics that include later tokens; and tokens that a one-query decode
 * at the query's own fill level would read unquantised from the ring are
 * read quantised once a later flush has encoded them. Row i therefore equals
 * kvq_decode_attention over the first tokens - n_queries + i + 1 tokens
 * exactly when both fill levels quantise the same tokens,
 * q(tokens - n_queries + i + 1) == q(tokens), and differs slightly otherwise.
 *   n_queries  1 <= n_queries <= tokens (else KVQ_ERR_INVALID); 1 is exactly
 *              kvq_decode_attention; batch * n_queries <= 65535 (one row of
 *              blocks per (sequence, query); else KVQ_ERR_UNSUPPORTED)
 *   q          device [batch][n_queries][q_heads][head_dim], q_dtype
 *   out        device fp32 [batch][n_queries][q_heads][head_dim]
 *   workspace  >= n_queries * kvq_cache_bytes(cfg, tokens, KVQ_BYTES_WORKSPACE),
 *              zero-filled before first use (as for kvq_decode_attention)
 * Other arguments, requirements and errors as kvq_decode_attention. With
 * n_queries > 1, KIVI caches of 16-bit inputs run on the matrix-core kernel,
 * one row of blocks per query (a query whose token is in a quantised page
 * sees that page masked after its token), or, at GQA 4 without rotary keys
 * and with an even n_queries whose tokens are all in the ring, one row of
 * blocks per two consecutive queries that share every page; FP8 and bfloat16
 * caches without in-kernel rotary embedding (head_dim >= 64) run on their
 * matrix-core kernel; every other case runs on the generic (vector-ALU)
 * kernel. */
KVQ_API int32_t kvq_decode_attention_multi(const kvq_config* cfg, const void* cache,
                                   int32_t layer, int64_t tokens, int32_t n_queries,
                                   const void* q, const float* k_scale,
                                   const float* v_scale, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Size of the library's own decode scratch array, per GPU (see
 * kvq_decode_attention_noalloc). */
#define KVQ_NOALLOC_SCRATCH_BYTES (16 << 20)

/* kvq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * forbid allocation. Same arguments (minus workspace), same kernels, same
 * result bit for bit as kvq_decode_attention with a workspace of
 * kvq_cache_bytes(cfg, tokens, KVQ_BYTES_WORKSPACE) bytes.
 *   The split partials and arrival counters live in a fixed device array of
 *   KVQ_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 *   until the process ends. A call whose workspace need exceeds it returns
 *   KVQ_ERR_WORKSPACE (validated on the host, nothing launched). The call
 *   allocates nothing. The first call on a device looks up the array's
 *   address and enqueues one small kernel on `stream` that clears it; every
 *   decode leaves its counters and partials at zero again.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (different streams, or concurrent graph replays) race and give
 *   wrong results; serialise them, or use kvq_decode_attention with a
 *   workspace of its own per stream. */
KVQ_API int32_t kvq_decode_attention_noalloc(const kvq_config* cfg, const void* cache,
                                     int32_t layer, int64_t tokens, const void* q,
                                     const float* k_scale, const float* v_scale,
                                     float* out, void* stream);

/* Static description of a status code (never NULL). */
KVQ_API const char* kvq_status_string(int32_t status);

/* KVQ_ABI_VERSION of the built library. */
KVQ_API int32_t kvq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
