// Generic decode kernel instances: KIVI caches with 3-bit codes ("Quantising
// the Cache.", Twice the users for nearly nothing: the 3-bit cache; KVQuant
// Key points: 3-bit keys and values), keys or values or both.
#include "decode_generic.h"

namespace kvq {
namespace gen {

hipError_t run_kivi3(const DecodeParams& p, const Geometry& g, hipStream_t st) {
  if (g.bits == 3) {
    return g.vbits == 2 ? by_d<KVQ_KIVI, 3, 2>(p, g.d, g.hg, g.batch, st)
                        : by_d<KVQ_KIVI, 3, 3>(p, g.d, g.hg, g.batch, st);
  }
  return g.bits == 4 ? by_d<KVQ_KIVI, 4, 3>(p, g.d, g.hg, g.batch, st)
                     : by_d<KVQ_KIVI, 8, 3>(p, g.d, g.hg, g.batch, st);
}

}  // namespace gen
}  // namespace kvq
