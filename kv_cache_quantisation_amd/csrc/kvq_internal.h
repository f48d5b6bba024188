// Internal geometry of the cache layout and kernel launch interfaces.
// Layout v1 is specified in include/kvq.h; this is the library's own
// computation of its offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kPage = 32;  // tokens per page == KIVI key group

// Either FP8 format: one byte per value, per-(layer, KV head) scales.
__host__ __device__ constexpr bool is_fp8(int scheme) {
  return scheme == KVQ_FP8_E4M3 || scheme == KVQ_FP8_E5M2;
}
// Schemes whose keys take the per-head static key scale (FP8 keys).
__host__ __device__ constexpr bool has_key_scale(int scheme) {
  return is_fp8(scheme) || scheme == KVQ_FP8K_SYMV || scheme == KVQ_FP8K_KIVIV;
}
// FP8 keys with values of another cache type (symmetric or KIVI, per token).
__host__ __device__ constexpr bool is_fp8_keys_mixed(int scheme) {
  return scheme == KVQ_FP8K_SYMV || scheme == KVQ_FP8K_KIVIV;
}

// Everything a kernel needs to address one layer of the cache.
struct Geometry {
  int32_t scheme, bits, d, hg, kv_heads, q_heads, batch, layers, residual;
  int32_t vbits;            // bits of the value codes (KIVI; = bits otherwise)
  int32_t in_bytes;         // bytes per K/V input element (and ring element)
  double rope;              // rotary base (0 = none)
  int64_t capacity;         // max_tokens
  int64_t page_bytes;       // bytes of one 32-token page
  int64_t pages_per_slab;   // P
  int64_t ring_slots;       // R + 32 (KIVI), else 0
  int64_t ring_bytes;       // 2 * ring_slots * d * in_bytes
  int64_t slab_bytes;       // P * page_bytes + ring_bytes
  // byte offsets inside a page
  int32_t off_kc, off_ks, off_kz, off_vc, off_vs, off_vz;
  // dense-and-sparse KIVI pages: one outlier per vector in the side matrix
  int32_t outliers;
  int32_t off_ko, off_vo, off_ki, off_vi;   // -1 without outliers
};

// Fills g from a validated config. Returns KVQ_OK or a negative status.
int32_t make_geometry(const kvq_config& cfg, Geometry* g);

// Where the pages and the residual ring of (sequence b, KV head h) of one
// layer live. Slab layout (table == null): one contiguous slab per (sequence,
// KV head), its pages then its ring. Paged layout: a block table maps page p
// of sequence b to a physical block of the layer's pool (each block one page
// per KV head) and the rings sit in their own region, one per (sequence, KV
// head); block numbers are clamped into the pool so that every access stays
// inside the caller's buffer.
struct PageMap {
  uint8_t* base;            // slab layout: the layer's first slab; paged: its first block
  uint8_t* rings;           // paged: the layer's first ring
  const int32_t* table;     // paged: [batch][max_blocks] block numbers, else null
  int64_t unit_bytes;       // slab layout: bytes per slab; paged: bytes per ring
  int64_t ring_off;         // slab layout: offset of the ring inside a slab
  int64_t page_bytes;
  int32_t kv_heads, max_blocks, num_blocks;

  __device__ __forceinline__ uint8_t* page(int b, int h, int64_t p) const {
    if (table) {
      int32_t id = table[static_cast<int64_t>(b) * max_blocks + p];
      id = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
      return base + (static_cast<int64_t>(id) * kv_heads + h) * page_bytes;
    }
    return base + (static_cast<int64_t>(b) * kv_heads + h) * unit_bytes + p * page_bytes;
  }
  __device__ __forceinline__ uint8_t* ring(int b, int h) const {
    if (table) return rings + (static_cast<int64_t>(b) * kv_heads + h) * unit_bytes;
    return base + (static_cast<int64_t>(b) * kv_heads + h) * unit_bytes + ring_off;
  }
};

// Bytes of the ring region of a paged cache (all layers), 256-aligned.
int64_t paged_ring_region(const Geometry& g);
// Bytes of a paged cache with num_blocks blocks per layer, or -1 on overflow.
int64_t paged_cache_bytes(const Geometry& g, int64_t num_blocks);

// Page map of `layer` of a cache buffer: the slab layout (table null) or the
// paged one.
PageMap make_page_map(const Geometry& g, const uint8_t* cache, int32_t layer,
                      const int32_t* table, int32_t max_blocks, int64_t num_blocks);

// Tokens sequence b holds (its own fill level in a ragged batch): seq[b]
// clamped to [1, T], or T without seq.
__device__ inline int64_t seq_len(const int64_t* seq, int b, int64_t T) {
  if (!seq) return T;
  const int64_t t = seq[b];
  return t < 1 ? 1 : (t > T ? T : t);
}

// Number of quantised tokens of a KIVI cache holding T tokens.
__host__ __device__ inline int64_t kivi_quantised(int64_t T, int32_t R) {
  const int64_t over = T - R;
  return over > 0 ? (over / kPage) * kPage : 0;
}

// ---- launch interfaces (implemented in append.hip / decode.hip) ----------

struct AppendArgs {
  Geometry g;
  PageMap pm;               // where this layer's pages and rings are
  uint8_t* layer_base;      // cache + layer * batch * kv_heads * slab_bytes (slab layout)
  const void* k_new;        // [B][n][Hkv][d] in_dtype
  const void* v_new;
  const float* k_scale;     // FP8 only
  const float* v_scale;
  int64_t past, n;          // tokens before the call, tokens appended
  const int64_t* seq_past;  // ragged batch: per-sequence past / appended counts (device),
  const int64_t* seq_new;   //   or null; n is then the bound (input rows per sequence)
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct DecodeArgs {
  Geometry g;
  PageMap pm;               // where this layer's pages and rings are
  const uint8_t* layer_base;
  int64_t tokens;
  const int64_t* seq_tokens;  // device [B] per-sequence token counts, or null (all = tokens)
  int32_t nq;               // queries per sequence (0 or 1: one; > 1: causal)
  const void* q;            // [B][Hq][d] q_dtype
  int32_t q_dtype;
  const float* k_scale;     // FP8 only
  const float* v_scale;
  float* out;               // [B][Hq][d]
  uint8_t* workspace;
  float sm_scale;           // resolved (never 0)
  double rope_theta;        // 0 = off
  int32_t splits;           // token splits per (seq, KV head), >= 1
  int32_t items;            // work items (pages + ring chunks) per (seq, KV head)
  int32_t requested_splits; // cfg.num_splits
  const void* k_new;        // fused one-token append: the token at position tokens - 1,
  const void* v_new;        //   [batch][kv_heads][d] in_dtype (null: none)
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Matrix-core path: KIVI 2/4-bit pages, head_dim >= 64, no rotary embedding.
// Blocks [0, page_splits) take page ranges; ring_splits more take ring chunks.
struct MfmaPlan {
  int32_t pages, chunks, page_splits, ring_splits, ring_splits_max;
};
bool mfma_path(const Geometry& g);
// Several queries (nq) of a uniform batch on the KIVI matrix-core kernel
// (mfma_path; queries whose tokens are in pages see a masked last page).
bool mfma_multi_ok(const Geometry& g, int64_t tokens, int32_t nq);
MfmaPlan mfma_plan(const Geometry& g, int64_t tokens, int32_t requested);
hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t stream);
// The matrix-core KIVI kernel takes a fused one-token append (kivi_mfma_kernel,
// not the rotary GQA-4 kernel).
bool mfma_fused_append_ok(const Geometry& g);
// Matrix-core path of FP8 E4M3 and bfloat16 caches (head_dim >= 64, no rotary embedding).
bool fp8_mfma_path(const Geometry& g);
int32_t fp8_mfma_splits(const Geometry& g, int64_t tokens, int32_t requested);
hipError_t launch_fp8_mfma(const DecodeArgs& a, hipStream_t stream);

// Decode split plan, shared by kvq_cache_bytes(WORKSPACE) and the launcher.
int32_t decode_items(const Geometry& g, int64_t tokens);
int32_t decode_splits(const Geometry& g, int64_t tokens, int32_t requested);
int64_t workspace_bytes_for(const Geometry& g, int64_t tokens, int32_t requested);
// Validates a decode call (nothing touches a device) and fills its launch
// arguments; KVQ_OK or the negative status the entry point returns.
int32_t decode_prepare(const kvq_config* cfg, const void* cache, int32_t layer, int64_t tokens,
                       const int64_t* seq_tokens, int32_t nq, const void* q,
                       const float* k_scale, const float* v_scale, float* out, void* workspace,
                       size_t workspace_bytes, DecodeArgs* args,
                       const int32_t* table = nullptr, int32_t max_blocks = 0,
                       int64_t num_blocks = 0);
// Offset of the split partials inside the workspace (after the counters).
int64_t workspace_partials_offset(const Geometry& g);

}  // namespace kvq
