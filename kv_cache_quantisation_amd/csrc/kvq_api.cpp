// Host side of the C ABI: argument validation, cache geometry, byte counts
// and kernel dispatch. Nothing here touches a device before validation has
// passed, so every error path can be exercised without a GPU.
#include <cmath>
#include <cstdint>
#include <limits>

#include "kvq_internal.h"

namespace kvq {
namespace {

bool is_pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

// Multiplies non-negative int64 values, returning -1 on overflow.
int64_t mul_ck(int64_t a, int64_t b) {
  if (a < 0 || b < 0) return -1;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return -1;
  return a * b;
}

int32_t validate_config(const kvq_config* cfg) {
  if (!cfg) return KVQ_ERR_NULL;
  if (cfg->struct_size != sizeof(kvq_config)) return KVQ_ERR_INVALID;
  const kvq_config& c = *cfg;
  if (c.scheme != KVQ_KIVI && c.scheme != KVQ_SYM_TOKEN && c.scheme != KVQ_FP8_E4M3 &&
      c.scheme != KVQ_FP8_E5M2 && c.scheme != KVQ_BF16_CACHE && c.scheme != KVQ_FP8K_SYMV &&
      c.scheme != KVQ_FP8K_KIVIV)
    return KVQ_ERR_INVALID;
  if (kvq::is_fp8_keys_mixed(c.scheme)) {   // FP8 keys, symmetric or KIVI values at v_bits
    if (c.bits != 8) return KVQ_ERR_INVALID;
    if (c.v_bits != 0 && (c.v_bits < 1 || c.v_bits > 8)) return KVQ_ERR_INVALID;
    if (c.v_bits != 0 && c.v_bits != 2 && c.v_bits != 3 && c.v_bits != 4 && c.v_bits != 8)
      return KVQ_ERR_UNSUPPORTED;
    if (c.v_bits == 3 && c.head_dim < 64) return KVQ_ERR_UNSUPPORTED;
  } else if (c.scheme == KVQ_FP8_E4M3 || c.scheme == KVQ_FP8_E5M2) {
    if (c.bits != 8) return KVQ_ERR_INVALID;
  } else if (c.scheme == KVQ_BF16_CACHE) {
    if (c.bits != 16) return KVQ_ERR_INVALID;
  } else if (c.bits != 2 && c.bits != 3 && c.bits != 4 && c.bits != 8) {
    return (c.bits >= 1 && c.bits <= 8) ? KVQ_ERR_UNSUPPORTED : KVQ_ERR_INVALID;
  }
  if (c.v_bits != 0 && c.v_bits != c.bits && !kvq::is_fp8_keys_mixed(c.scheme)) {
    if (c.scheme != KVQ_KIVI || c.v_bits < 1 || c.v_bits > 8) return KVQ_ERR_INVALID;
    if ((c.v_bits != 2 && c.v_bits != 3 && c.v_bits != 4) || c.v_bits > c.bits)
      return KVQ_ERR_UNSUPPORTED;
    // 3 bits next to another width: pages stay 256-byte multiples from d = 64
    if ((c.bits == 3 || c.v_bits == 3) && c.head_dim < 64) return KVQ_ERR_UNSUPPORTED;
  }
  if (c.outliers != 0 && (c.outliers != 1 || c.scheme != KVQ_KIVI)) return KVQ_ERR_INVALID;
  if (c.layers < 1 || c.q_heads < 1 || c.kv_heads < 1 || c.batch < 1 || c.max_tokens < 0)
    return KVQ_ERR_INVALID;
  if (c.q_heads % c.kv_heads != 0) return KVQ_ERR_INVALID;
  // grid limits: (splits, kv_heads, batch); page counts fit in int32
  if (c.kv_heads > 65535 || c.batch > 65535 || c.max_tokens >= (int64_t(1) << 36))
    return KVQ_ERR_UNSUPPORTED;
  if (!is_pow2_in(c.q_heads / c.kv_heads, 1, 8)) return KVQ_ERR_UNSUPPORTED;
  if (c.head_dim < 1) return KVQ_ERR_INVALID;
  if (!is_pow2_in(c.head_dim, 32, 256)) return KVQ_ERR_UNSUPPORTED;
  if (c.group < 1) return KVQ_ERR_INVALID;
  if (c.group != kPage) return KVQ_ERR_UNSUPPORTED;
  if (c.residual < 0) return KVQ_ERR_INVALID;
  if (c.scheme != KVQ_KIVI && c.residual != 0) return KVQ_ERR_INVALID;
  if (c.in_dtype != KVQ_F32 && c.in_dtype != KVQ_BF16) return KVQ_ERR_INVALID;
  if (c.q_dtype != KVQ_F32 && c.q_dtype != KVQ_BF16) return KVQ_ERR_INVALID;
  if (!std::isfinite(c.rope_theta) || c.rope_theta < 0) return KVQ_ERR_INVALID;
  if (!std::isfinite(c.sm_scale)) return KVQ_ERR_INVALID;
  if (c.num_splits < 0) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

int64_t slab_bytes_for(const Geometry& g, int64_t capacity) {
  const int64_t pages = g.scheme == KVQ_KIVI
                            ? (capacity > g.residual ? (capacity - g.residual) / kPage : 0)
                            : (capacity + kPage - 1) / kPage;
  const int64_t p = mul_ck(pages, g.page_bytes);
  if (p < 0) return -1;
  return p + g.ring_bytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int32_t make_geometry(const kvq_config& c, Geometry* g) {
  const int32_t st = validate_config(&c);
  if (st != KVQ_OK) return st;
  Geometry x{};
  x.off_ko = x.off_vo = x.off_ki = x.off_vi = -1;
  x.scheme = c.scheme;
  x.bits = c.bits;
  x.vbits = c.v_bits != 0 ? c.v_bits : c.bits;
  x.d = c.head_dim;
  x.hg = c.q_heads / c.kv_heads;
  x.kv_heads = c.kv_heads;
  x.q_heads = c.q_heads;
  x.batch = c.batch;
  x.layers = c.layers;
  x.residual = c.residual;
  x.in_bytes = c.in_dtype == KVQ_BF16 ? 2 : 4;
  x.rope = c.rope_theta;
  x.capacity = c.max_tokens;
  const int32_t d = c.head_dim, b = c.bits;
  const int32_t codes = kPage * d * b / 8;  // one packed K-rows or V-cols run
  const int32_t vcodes = kPage * d * x.vbits / 8;   // KIVI value codes
  switch (c.scheme) {
    case KVQ_KIVI:
      x.off_kc = 0;
      x.off_ks = codes;
      x.off_kz = codes + 4 * d;
      x.off_vc = codes + 8 * d;
      x.off_vs = codes + vcodes + 8 * d;
      x.off_vz = codes + vcodes + 8 * d + 4 * kPage;
      x.page_bytes = codes + vcodes + 8 * d + 8 * kPage;
      x.ring_slots = c.residual + kPage;
      if (c.outliers) {   // side matrix after the dense page, padded to 256 bytes
        x.outliers = 1;
        x.off_ko = static_cast<int32_t>(x.page_bytes);
        x.off_vo = x.off_ko + 4 * d;
        x.off_ki = x.off_vo + 4 * kPage;
        x.off_vi = x.off_ki + d;
        x.page_bytes += (5 * d + 5 * kPage + 255) / 256 * 256;
      }
      break;
    case KVQ_SYM_TOKEN:
      x.off_kc = 0;
      x.off_ks = codes;
      x.off_vc = codes + 4 * kPage;
      x.off_vs = 2 * codes + 4 * kPage;
      x.off_kz = x.off_vz = -1;
      x.page_bytes = 2 * codes + 8 * kPage;
      x.ring_slots = 0;
      break;
    case KVQ_FP8K_SYMV:   // FP8 K rows, symmetric V cols, V scales (padded to 256 bytes)
      x.off_kc = 0;
      x.off_vc = codes;
      x.off_vs = codes + vcodes;
      x.off_ks = x.off_kz = x.off_vz = -1;
      x.page_bytes = codes + vcodes + 256;
      x.ring_slots = 0;
      break;
    case KVQ_FP8K_KIVIV:   // FP8 K rows, KIVI V cols, V scale and offset per token
      x.off_kc = 0;
      x.off_vc = codes;
      x.off_vs = codes + vcodes;
      x.off_vz = codes + vcodes + 4 * kPage;
      x.off_ks = x.off_kz = -1;
      x.page_bytes = codes + vcodes + 8 * kPage;
      x.ring_slots = 0;
      break;
    default:  // FP8, either format (b = 8), and BF16_CACHE (b = 16): K rows, then V cols
      x.off_kc = 0;
      x.off_vc = codes;
      x.off_ks = x.off_kz = x.off_vs = x.off_vz = -1;
      x.page_bytes = 2 * codes;
      x.ring_slots = 0;
      break;
  }
  x.ring_bytes = 2 * x.ring_slots * d * x.in_bytes;
  x.pages_per_slab = x.scheme == KVQ_KIVI
                         ? (c.max_tokens > c.residual ? (c.max_tokens - c.residual) / kPage : 0)
                         : (c.max_tokens + kPage - 1) / kPage;
  x.slab_bytes = slab_bytes_for(x, c.max_tokens);
  if (x.slab_bytes < 0) return KVQ_ERR_INVALID;
  const int64_t slabs = mul_ck(mul_ck(c.layers, c.batch), c.kv_heads);
  if (mul_ck(slabs, x.slab_bytes) < 0) return KVQ_ERR_INVALID;
  *g = x;
  return KVQ_OK;
}

int64_t paged_ring_region(const Geometry& g) {
  const int64_t r = mul_ck(mul_ck(mul_ck(g.layers, g.batch), g.kv_heads), g.ring_bytes);
  return r < 0 ? -1 : (r + 255) / 256 * 256;
}

int64_t paged_cache_bytes(const Geometry& g, int64_t num_blocks) {
  const int64_t rings = paged_ring_region(g);
  const int64_t blocks = mul_ck(mul_ck(mul_ck(g.layers, num_blocks), g.kv_heads), g.page_bytes);
  if (rings < 0 || blocks < 0 || blocks > std::numeric_limits<int64_t>::max() - rings) return -1;
  return rings + blocks;
}

PageMap make_page_map(const Geometry& g, const uint8_t* cache, int32_t layer,
                      const int32_t* table, int32_t max_blocks, int64_t num_blocks) {
  PageMap m{};
  uint8_t* c = const_cast<uint8_t*>(cache);
  m.page_bytes = g.page_bytes;
  m.kv_heads = g.kv_heads;
  if (!table) {
    m.base = c + static_cast<int64_t>(layer) * g.batch * g.kv_heads * g.slab_bytes;
    m.unit_bytes = g.slab_bytes;
    m.ring_off = g.pages_per_slab * g.page_bytes;
    return m;
  }
  m.table = table;
  m.max_blocks = max_blocks;
  m.num_blocks = static_cast<int32_t>(num_blocks);
  m.rings = c + static_cast<int64_t>(layer) * g.batch * g.kv_heads * g.ring_bytes;
  m.base = c + paged_ring_region(g) + static_cast<int64_t>(layer) * num_blocks * g.kv_heads * g.page_bytes;
  m.unit_bytes = g.ring_bytes;
  return m;
}

int32_t decode_items(const Geometry& g, int64_t tokens) {
  if (g.scheme == KVQ_KIVI) {
    const int64_t q = kivi_quantised(tokens, g.residual);
    const int64_t nr = tokens - q;
    return static_cast<int32_t>(q / kPage + (nr + kPage - 1) / kPage);
  }
  return static_cast<int32_t>((tokens + kPage - 1) / kPage);
}

int32_t decode_splits(const Geometry& g, int64_t tokens, int32_t requested) {
  const int64_t items = decode_items(g, tokens);
  if (items <= 0) return 1;
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    // Aim at ~1024 blocks on 256 CUs while keeping >= 8 work items per block.
    const int64_t units = static_cast<int64_t>(g.batch) * g.kv_heads;
    s = (1024 + units - 1) / units;
    const int64_t cap = (items + 7) / 8;
    if (s > cap) s = cap;
  }
  if (s > items) s = items;
  if (s < 1) s = 1;
  return static_cast<int32_t>(s);
}

int64_t workspace_partials_offset(const Geometry& g) {
  const int64_t counters = static_cast<int64_t>(g.batch) * g.kv_heads * 4;
  return (counters + 255) / 256 * 256;
}

// Split count of a one-query decode of this configuration (its workspace holds
// that many partials per (sequence, query head)).
int64_t single_splits(const Geometry& g, int64_t tokens, int32_t requested) {
  if (mfma_path(g)) {
    const MfmaPlan pl = mfma_plan(g, tokens, requested);
    return static_cast<int64_t>(pl.page_splits) + pl.ring_splits_max;
  }
  if (fp8_mfma_path(g)) return fp8_mfma_splits(g, tokens, requested);
  return decode_splits(g, tokens, requested);
}

int64_t workspace_bytes_for(const Geometry& g, int64_t tokens, int32_t requested) {
  const int64_t s = single_splits(g, tokens, requested);
  const int64_t per = static_cast<int64_t>(g.d + 2) * 4;
  int64_t p = mul_ck(mul_ck(mul_ck(g.batch, g.q_heads), s), per);
  if (p < 0) return -1;
  return workspace_partials_offset(g) + p;
}

}  // namespace kvq

using kvq::Geometry;

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(int32_t s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "cache capacity exceeded";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t kvq_cache_bytes(const kvq_config* cfg, int64_t tokens, int32_t kind) {
  if (!cfg) return KVQ_ERR_NULL;
  Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  if (tokens < 0) return KVQ_ERR_INVALID;
  if (tokens >= (int64_t(1) << 36)) return KVQ_ERR_UNSUPPORTED;
  switch (kind) {
    case KVQ_BYTES_FORMULA: {
      // batch * layers * kv_heads * head_dim * tokens * (key bits + value bits) / 8
      int64_t v = kvq::mul_ck(cfg->batch, cfg->layers);
      v = kvq::mul_ck(v, cfg->kv_heads);
      v = kvq::mul_ck(v, cfg->head_dim);
      v = kvq::mul_ck(v, tokens);
      v = kvq::mul_ck(v, g.bits + g.vbits);
      return v < 0 ? KVQ_ERR_INVALID : v / 8;
    }
    case KVQ_BYTES_CACHE: {
      const int64_t slab = kvq::slab_bytes_for(g, tokens);
      int64_t v = kvq::mul_ck(kvq::mul_ck(kvq::mul_ck(cfg->layers, cfg->batch), cfg->kv_heads),
                              slab);
      return (slab < 0 || v < 0) ? KVQ_ERR_INVALID : v;
    }
    case KVQ_BYTES_WORKSPACE: {
      const int64_t v = kvq::workspace_bytes_for(g, tokens, cfg->num_splits);
      return v < 0 ? KVQ_ERR_INVALID : v;
    }
    default:
      return KVQ_ERR_INVALID;
  }
}

int32_t kvq_quantize_append(const kvq_config* cfg, void* cache, int32_t layer,
                            int64_t past_tokens, int64_t new_tokens, const void* k_new,
                            const void* v_new, const float* k_scale, const float* v_scale,
                            void* stream) {
  if (!cfg) return KVQ_ERR_NULL;
  Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  if (!cache) return KVQ_ERR_NULL;
  if (layer < 0 || layer >= cfg->layers) return KVQ_ERR_INVALID;
  if (past_tokens < 0 || new_tokens < 0) return KVQ_ERR_INVALID;
  if (past_tokens > cfg->max_tokens || new_tokens > cfg->max_tokens - past_tokens)
    return KVQ_ERR_CAPACITY;
  if (new_tokens == 0) return KVQ_OK;
  if (!k_new || !v_new) return KVQ_ERR_NULL;
  if (kvq::has_key_scale(cfg->scheme) && !k_scale) return KVQ_ERR_NULL;
  if (kvq::is_fp8(cfg->scheme) && !v_scale) return KVQ_ERR_NULL;
  if (!kvq::aligned16(cache) || !kvq::aligned16(k_new) || !kvq::aligned16(v_new))
    return KVQ_ERR_INVALID;
  kvq::AppendArgs a{};
  a.g = g;
  a.pm = kvq::make_page_map(g, static_cast<uint8_t*>(cache), layer, nullptr, 0, 0);
  a.layer_base = static_cast<uint8_t*>(cache) +
                 static_cast<int64_t>(layer) * cfg->batch * cfg->kv_heads * g.slab_bytes;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.past = past_tokens;
  a.n = new_tokens;
  const hipError_t e = kvq::launch_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

}  // extern "C"

namespace {
// Ragged quantize-append into the slab layout (table null) or a paged cache.
int32_t append_ragged(const kvq_config* cfg, void* cache, int32_t layer, const int32_t* table,
                      int32_t max_blocks, int64_t num_blocks, const int64_t* seq_past,
                      const int64_t* seq_new, int64_t new_max, const void* k_new,
                      const void* v_new, const float* k_scale, const float* v_scale,
                      void* stream) {
  if (!cfg) return KVQ_ERR_NULL;
  Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  if (!cache) return KVQ_ERR_NULL;
  if (layer < 0 || layer >= cfg->layers) return KVQ_ERR_INVALID;
  if (new_max < 0) return KVQ_ERR_INVALID;
  if (new_max > cfg->max_tokens) return KVQ_ERR_CAPACITY;
  if (new_max == 0) return KVQ_OK;
  if (!seq_past || !seq_new || !k_new || !v_new) return KVQ_ERR_NULL;
  if (kvq::has_key_scale(cfg->scheme) && !k_scale) return KVQ_ERR_NULL;
  if (kvq::is_fp8(cfg->scheme) && !v_scale) return KVQ_ERR_NULL;
  if (!kvq::aligned16(cache) || !kvq::aligned16(k_new) || !kvq::aligned16(v_new) ||
      (reinterpret_cast<uintptr_t>(seq_past) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(seq_new) & 7u) != 0)
    return KVQ_ERR_INVALID;
  kvq::AppendArgs a{};
  a.g = g;
  a.pm = kvq::make_page_map(g, static_cast<uint8_t*>(cache), layer, table, max_blocks, num_blocks);
  a.layer_base = static_cast<uint8_t*>(cache) +
                 static_cast<int64_t>(layer) * cfg->batch * cfg->kv_heads * g.slab_bytes;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.past = 0;
  a.n = new_max;
  a.seq_past = seq_past;
  a.seq_new = seq_new;
  const hipError_t e = kvq::launch_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

// Validates a block table's arguments against the configuration.
int32_t check_table(const kvq_config* cfg, const kvq::Geometry& g, const int32_t* table,
                    int32_t max_blocks, int64_t num_blocks) {
  if (!table) return KVQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(table) & 3u) != 0) return KVQ_ERR_INVALID;
  if (max_blocks < 1 || num_blocks < 1) return KVQ_ERR_INVALID;
  if (num_blocks > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  if (max_blocks < g.pages_per_slab) return KVQ_ERR_CAPACITY;   // a full sequence's pages
  (void)cfg;
  return kvq::paged_cache_bytes(g, num_blocks) < 0 ? KVQ_ERR_INVALID : KVQ_OK;
}
}  // namespace

extern "C" {

int32_t kvq_quantize_append_ragged(const kvq_config* cfg, void* cache, int32_t layer,
                                   const int64_t* seq_past, const int64_t* seq_new,
                                   int64_t new_max, const void* k_new, const void* v_new,
                                   const float* k_scale, const float* v_scale, void* stream) {
  return append_ragged(cfg, cache, layer, nullptr, 0, 0, seq_past, seq_new, new_max, k_new,
                       v_new, k_scale, v_scale, stream);
}

int32_t kvq_quantize_append_paged(const kvq_config* cfg, void* cache, int32_t layer,
                                  const int32_t* block_table, int32_t max_blocks,
                                  int64_t num_blocks, const int64_t* seq_past,
                                  const int64_t* seq_new, int64_t new_max, const void* k_new,
                                  const void* v_new, const float* k_scale, const float* v_scale,
                                  void* stream) {
  if (!cfg) return KVQ_ERR_NULL;
  kvq::Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  const int32_t tst = check_table(cfg, g, block_table, max_blocks, num_blocks);
  if (tst != KVQ_OK) return tst;
  return append_ragged(cfg, cache, layer, block_table, max_blocks, num_blocks, seq_past, seq_new,
                       new_max, k_new, v_new, k_scale, v_scale, stream);
}

int64_t kvq_paged_cache_bytes(const kvq_config* cfg, int64_t num_blocks) {
  if (!cfg) return KVQ_ERR_NULL;
  kvq::Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  if (num_blocks < 0) return KVQ_ERR_INVALID;
  if (num_blocks > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  const int64_t v = kvq::paged_cache_bytes(g, num_blocks);
  return v < 0 ? KVQ_ERR_INVALID : v;
}

}  // extern "C"

namespace kvq {
// Validation of a decode call and its launch arguments (no device access).
int32_t decode_prepare(const kvq_config* cfg, const void* cache, int32_t layer, int64_t tokens,
                       const int64_t* seq_tokens, int32_t nq, const void* q,
                       const float* k_scale, const float* v_scale, float* out, void* workspace,
                       size_t workspace_bytes, DecodeArgs* args, const int32_t* table,
                       int32_t max_blocks, int64_t num_blocks) {
  if (!cfg) return KVQ_ERR_NULL;
  Geometry g;
  const int32_t st = make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  if (!cache || !q || !out || !workspace) return KVQ_ERR_NULL;
  if (has_key_scale(cfg->scheme) && !k_scale) return KVQ_ERR_NULL;
  if (is_fp8(cfg->scheme) && !v_scale) return KVQ_ERR_NULL;
  if (layer < 0 || layer >= cfg->layers) return KVQ_ERR_INVALID;
  if (tokens < 1) return KVQ_ERR_INVALID;
  if (tokens > cfg->max_tokens) return KVQ_ERR_CAPACITY;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return KVQ_ERR_INVALID;
  if (nq < 1 || nq > tokens) return KVQ_ERR_INVALID;
  // one row of blocks per (sequence, query): the grid's z dimension
  if (static_cast<int64_t>(cfg->batch) * nq > 65535) return KVQ_ERR_UNSUPPORTED;
  const int64_t one = workspace_bytes_for(g, tokens, cfg->num_splits);
  if (one < 0) return KVQ_ERR_INVALID;
  if (workspace_bytes / static_cast<size_t>(nq) < static_cast<size_t>(one)) return KVQ_ERR_WORKSPACE;
  DecodeArgs a{};
  a.g = g;
  a.pm = make_page_map(g, static_cast<const uint8_t*>(cache), layer, table, max_blocks, num_blocks);
  a.layer_base = static_cast<const uint8_t*>(cache) +
                 static_cast<int64_t>(layer) * cfg->batch * cfg->kv_heads * g.slab_bytes;
  a.tokens = tokens;
  a.seq_tokens = seq_tokens;
  a.nq = nq;
  a.q = q;
  a.q_dtype = cfg->q_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.workspace = static_cast<uint8_t*>(workspace);
  a.sm_scale = cfg->sm_scale != 0.0f ? cfg->sm_scale
                                     : static_cast<float>(1.0 / std::sqrt((double)cfg->head_dim));
  a.rope_theta = cfg->rope_theta;
  a.items = decode_items(g, tokens);
  a.splits = decode_splits(g, tokens, cfg->num_splits);
  // several queries: the generic kernel takes the one-query split count (the
  // matrix-core kernels plan theirs for batch * n_queries rows, never more),
  // so that n_queries one-query workspaces hold the partials
  if (nq > 1) a.splits = static_cast<int32_t>(single_splits(g, tokens, cfg->num_splits));
  a.requested_splits = cfg->num_splits;
  *args = a;
  return KVQ_OK;
}
}  // namespace kvq

namespace {
int32_t decode_call(const kvq_config* cfg, const void* cache, int32_t layer, int64_t tokens,
                    const int64_t* seq_tokens, int32_t nq, const void* q, const float* k_scale,
                    const float* v_scale, float* out, void* workspace, size_t workspace_bytes,
                    void* stream, const int32_t* table = nullptr, int32_t max_blocks = 0,
                    int64_t num_blocks = 0) {
  kvq::DecodeArgs a;
  const int32_t st = kvq::decode_prepare(cfg, cache, layer, tokens, seq_tokens, nq, q, k_scale,
                                         v_scale, out, workspace, workspace_bytes, &a, table,
                                         max_blocks, num_blocks);
  if (st != KVQ_OK) return st;
  const hipError_t e = kvq::launch_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}
}  // namespace

extern "C" {

int32_t kvq_decode_attention(const kvq_config* cfg, const void* cache, int32_t layer,
                             int64_t tokens, const void* q, const float* k_scale,
                             const float* v_scale, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_call(cfg, cache, layer, tokens, nullptr, 1, q, k_scale, v_scale, out, workspace,
                     workspace_bytes, stream);
}

int32_t kvq_append_decode(const kvq_config* cfg, void* cache, int32_t layer, int64_t past_tokens,
                          const void* k_new, const void* v_new, const float* k_scale,
                          const float* v_scale, const void* q, float* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!cfg) return KVQ_ERR_NULL;
  if (past_tokens < 0) return KVQ_ERR_INVALID;
  if (past_tokens >= cfg->max_tokens) return KVQ_ERR_CAPACITY;
  // the decode's validation (over past_tokens + 1 tokens), then the append's
  kvq::DecodeArgs a;
  const int32_t st = kvq::decode_prepare(cfg, cache, layer, past_tokens + 1, nullptr, 1, q, k_scale,
                                         v_scale, out, workspace, workspace_bytes, &a);
  if (st != KVQ_OK) return st;
  if (!k_new || !v_new) return KVQ_ERR_NULL;
  if (!kvq::aligned16(k_new) || !kvq::aligned16(v_new)) return KVQ_ERR_INVALID;
  const kvq::Geometry& g = a.g;
  const int64_t q_old = kvq::kivi_quantised(past_tokens, g.residual);
  const int64_t q_new = kvq::kivi_quantised(past_tokens + 1, g.residual);
  // one launch: a KIVI cache on the matrix-core kernel, the new token landing
  // in the ring (no page to encode); else the append's kernels, then the decode
  if (g.scheme == KVQ_KIVI && kvq::mfma_fused_append_ok(g) && q_new == q_old &&
      past_tokens >= q_new) {
    a.k_new = k_new;
    a.v_new = v_new;
    const hipError_t e = kvq::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
  }
  const int32_t ast = kvq_quantize_append(cfg, cache, layer, past_tokens, 1, k_new, v_new,
                                          k_scale, v_scale, stream);
  if (ast != KVQ_OK) return ast;
  const hipError_t e = kvq::launch_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

int32_t kvq_decode_attention_multi(const kvq_config* cfg, const void* cache, int32_t layer,
                                   int64_t tokens, int32_t n_queries, const void* q,
                                   const float* k_scale, const float* v_scale, float* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(cfg, cache, layer, tokens, nullptr, n_queries, q, k_scale, v_scale, out,
                     workspace, workspace_bytes, stream);
}

int32_t kvq_decode_attention_paged(const kvq_config* cfg, const void* cache, int32_t layer,
                                   const int32_t* block_table, int32_t max_blocks,
                                   int64_t num_blocks, int64_t tokens, const int64_t* seq_tokens,
                                   const void* q, const float* k_scale, const float* v_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!cfg) return KVQ_ERR_NULL;
  kvq::Geometry g;
  const int32_t st = kvq::make_geometry(*cfg, &g);
  if (st != KVQ_OK) return st;
  const int32_t tst = check_table(cfg, g, block_table, max_blocks, num_blocks);
  if (tst != KVQ_OK) return tst;
  if (!seq_tokens) return KVQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(seq_tokens) & 7u) != 0) return KVQ_ERR_INVALID;
  return decode_call(cfg, cache, layer, tokens, seq_tokens, 1, q, k_scale, v_scale, out,
                     workspace, workspace_bytes, stream, block_table, max_blocks, num_blocks);
}

int32_t kvq_decode_attention_ragged(const kvq_config* cfg, const void* cache, int32_t layer,
                                    int64_t tokens, const int64_t* seq_tokens, const void* q,
                                    const float* k_scale, const float* v_scale, float* out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!seq_tokens) return KVQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(seq_tokens) & 7u) != 0)
    return KVQ_ERR_INVALID;
  return decode_call(cfg, cache, layer, tokens, seq_tokens, 1, q, k_scale, v_scale, out,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"
