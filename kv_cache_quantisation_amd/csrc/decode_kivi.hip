// Generic decode kernel instances: KIVI caches with 2-, 4- or 8-bit codes
// (values at their own width) that the matrix-core kernels do not take.
#include "decode_generic.h"

namespace kvq {
namespace gen {

hipError_t run_kivi(const DecodeParams& p, const Geometry& g, hipStream_t st) {
  switch (g.bits) {
    case 2: return by_d<KVQ_KIVI, 2>(p, g.d, g.hg, g.batch, st);
    case 4:
      return g.vbits == 2 ? by_d<KVQ_KIVI, 4, 2>(p, g.d, g.hg, g.batch, st)
                          : by_d<KVQ_KIVI, 4>(p, g.d, g.hg, g.batch, st);
    default:
      return g.vbits == 2   ? by_d<KVQ_KIVI, 8, 2>(p, g.d, g.hg, g.batch, st)
             : g.vbits == 4 ? by_d<KVQ_KIVI, 8, 4>(p, g.d, g.hg, g.batch, st)
                            : by_d<KVQ_KIVI, 8>(p, g.d, g.hg, g.batch, st);
  }
}

}  // namespace gen
}  // namespace kvq
