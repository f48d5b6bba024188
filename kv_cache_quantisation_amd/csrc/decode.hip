// Decode attention: chooses the kernel of a call -- the matrix-core kernels
// (decode_mfma.hip: KIVI 2/4-bit pages of 16-bit inputs; decode_fp8.hip: FP8,
// bfloat16 and 2/4-bit per-token-code pages) where they apply, else the generic vector-ALU kernel
// (decode_generic.h) -- and fills its launch parameters.
#include <hip/hip_runtime.h>

#include "decode_generic.h"
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  // several queries per sequence: the matrix-core KIVI and FP8/bfloat16
  // kernels where they apply, else the generic kernel
  if (a.nq <= 1 && mfma_path(g)) return launch_kivi_mfma(a, st);
  if (a.nq > 1 && !a.seq_tokens && mfma_multi_ok(g, a.tokens, a.nq)) return launch_kivi_mfma(a, st);
  if (fp8_mfma_path(g) && (a.nq <= 1 || !a.seq_tokens)) return launch_fp8_mfma(a, st);
  gen::DecodeParams p{};
  p.pm = a.pm;
  p.layer_base = a.layer_base;
  p.q = static_cast<const uint8_t*>(a.q);
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.out = a.out;
  p.partials = reinterpret_cast<float*>(a.workspace + workspace_partials_offset(g));
  p.counters = reinterpret_cast<int*>(a.workspace);
  p.slab_bytes = g.slab_bytes;
  p.page_bytes = g.page_bytes;
  p.ring_base = g.pages_per_slab * g.page_bytes;
  p.ring_slots = g.ring_slots > 0 ? g.ring_slots : 1;
  p.T = a.tokens;
  p.seq_tokens = a.seq_tokens;
  p.residual = g.residual;
  p.nq = a.nq > 1 ? a.nq : 1;
  if (g.scheme == KVQ_KIVI) {
    p.q_tokens = kivi_quantised(a.tokens, g.residual);
    p.n_pages = static_cast<int32_t>(p.q_tokens / kPage);
  } else {
    p.q_tokens = a.tokens;
    p.n_pages = static_cast<int32_t>((a.tokens + kPage - 1) / kPage);
  }
  p.items = a.items;
  p.splits = a.splits;
  p.kv_heads = g.kv_heads;
  p.q_heads = g.q_heads;
  p.off_kc = g.off_kc;
  p.off_ks = g.off_ks;
  p.off_kz = g.off_kz;
  p.off_vc = g.off_vc;
  p.off_vs = g.off_vs;
  p.off_vz = g.off_vz;
  p.q_bf16 = a.q_dtype == KVQ_BF16;
  p.in_bf16 = g.in_bytes == 2;
  p.qscale = a.sm_scale * gen::kLog2e;
  p.rope_theta = a.rope_theta;
  p.outliers = g.outliers;
  p.off_ko = g.off_ko;
  p.off_vo = g.off_vo;
  p.off_ki = g.off_ki;
  p.off_vi = g.off_vi;
  if (g.scheme == KVQ_KIVI) {
    if (g.bits == 3 || g.vbits == 3) return gen::run_kivi3(p, g, st);
    return gen::run_kivi(p, g, st);
  }
  return gen::run_other(p, g, st);
}

}  // namespace kvq
