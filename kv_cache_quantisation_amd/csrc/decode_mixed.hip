// Generic decode kernel instances: FP8 E4M3 keys with values of another cache
// type ("Quantizing the KV cache", How the KV cache is quantized: separate key
// and value cache types), symmetric (FP8K_SYMV) or KIVI (FP8K_KIVIV) per-token
// value codes at 2, 3, 4 or 8 bits.
#include "decode_generic.h"

namespace kvq {
namespace gen {

template <int SCHEME>
hipError_t by_vbits(const DecodeParams& p, const Geometry& g, hipStream_t st) {
  switch (g.vbits) {
    case 2: return by_d<SCHEME, 8, 2>(p, g.d, g.hg, g.batch, st);
    case 3: return by_d<SCHEME, 8, 3>(p, g.d, g.hg, g.batch, st);
    case 4: return by_d<SCHEME, 8, 4>(p, g.d, g.hg, g.batch, st);
    default: return by_d<SCHEME, 8, 8>(p, g.d, g.hg, g.batch, st);
  }
}

hipError_t run_mixed(const DecodeParams& p, const Geometry& g, hipStream_t st) {
  return g.scheme == KVQ_FP8K_KIVIV ? by_vbits<KVQ_FP8K_KIVIV>(p, g, st)
                                    : by_vbits<KVQ_FP8K_SYMV>(p, g, st);
}

}  // namespace gen
}  // namespace kvq
