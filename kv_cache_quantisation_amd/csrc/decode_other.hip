// Generic decode kernel instances: symmetric per-token caches (2/3/4/8-bit),
// FP8 caches (E4M3, E5M2) and the bfloat16 cache, where the matrix-core
// kernels do not take them.
#include "decode_generic.h"

namespace kvq {
namespace gen {

hipError_t run_other(const DecodeParams& p, const Geometry& g, hipStream_t st) {
  switch (g.scheme) {
    case KVQ_SYM_TOKEN:
      switch (g.bits) {
        case 2: return by_d<KVQ_SYM_TOKEN, 2>(p, g.d, g.hg, g.batch, st);
        case 3: return by_d<KVQ_SYM_TOKEN, 3>(p, g.d, g.hg, g.batch, st);
        case 4: return by_d<KVQ_SYM_TOKEN, 4>(p, g.d, g.hg, g.batch, st);
        default: return by_d<KVQ_SYM_TOKEN, 8>(p, g.d, g.hg, g.batch, st);
      }
    case KVQ_BF16_CACHE:
      return by_d<KVQ_BF16_CACHE, 16>(p, g.d, g.hg, g.batch, st);
    case KVQ_FP8_E5M2:
      return by_d<KVQ_FP8_E5M2, 8>(p, g.d, g.hg, g.batch, st);
    case KVQ_FP8K_SYMV:
    case KVQ_FP8K_KIVIV:
      return run_mixed(p, g, st);
    default:
      return by_d<KVQ_FP8_E4M3, 8>(p, g.d, g.hg, g.batch, st);
  }
}

}  // namespace gen
}  // namespace kvq
