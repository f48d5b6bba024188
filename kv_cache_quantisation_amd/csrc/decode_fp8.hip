// Decode attention over FP8, bfloat16 and per-token-code caches on the matrix
// cores (gfx950).
//
// softmax(sm_scale q.K^T) V over the dequantised cache ("Quantizing the KV
// cache", going deeper; FP8 cache with a scale per KV head, "How the KV cache
// is quantized"). The dequantised key is e * ks_h and the value e * vs_h with
// e the E4M3 value of the stored byte, so the key scale folds into the query
// once per call and the value scale multiplies the output once:
//
//   scores: S^T[t][h] = sum_c e_tc (q_hc ks_h)   v_mfma_f32_16x16x32_f16,
//           A = E4M3 key bytes converted to f16 (exact), B = q' = q ks_h
//           split into an f16 high part (columns 0..HG-1) and remainder
//           (columns HG..2HG-1); B stays in registers for the whole call.
//   values: O[h][c] = vs_h sum_t p_ht e_tc       v_mfma_f32_16x16x32_bf16,
//           A = p in bf16 high/remainder rows, B = E4M3 value bytes converted
//           to bf16 (exact).
//
// Operand layouts (wave64): lane l holds A[l%16][8(l/16)+i], B[8(l/16)+i][l%16]
// and C[4(l/16)+r][l%16]. Key tile mt (0, 1) row rho holds token
// 8(rho/4) + 4 mt + rho%4 of the page, so lane (j, g) = (l%16, l/16) ends up
// with head j's scores for tokens 8g..8g+7 -- exactly the k-block of the P.V
// A operand, and the 8 value bytes of a channel it needs are contiguous.
//
// Pages (32 tokens, 64*d bytes) stream HBM -> LDS with global_load_lds_dwordx4,
// one page ahead of the one being computed. The last page of a cache may be
// partial: its absent tokens get score -inf and their value bytes are zeroed
// before conversion (unwritten bytes may hold E4M3 NaN patterns). Blocks of a
// (sequence, KV head) write partial (m, l, o); the last block to finish merges
// them and writes the output.
//
// The unquantised bfloat16 cache (the baseline the pages compare against)
// runs through the same kernel: its key rows are already bf16 and feed the
// key product directly (v_mfma_f32_16x16x32_bf16, q split into bf16 high and
// remainder), and only the key rows (64*d bytes per page) are staged in LDS;
// each lane loads the 16 value bytes it needs (8 tokens of one channel) from
// HBM straight into registers, one page ahead, so a page costs no more LDS
// than an FP8 page.
#include <hip/hip_runtime.h>

#include <type_traits>

#include <cmath>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_merge.h"
#include "kvq_wave.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct Fp8Params {
  const uint8_t* layer_base;
  const uint8_t* q;
  const float* k_scale;           // [kv_heads] of this layer
  const float* v_scale;
  float* out;
  float* partials;
  int* counters;                  // one per (sequence, KV head), zero between calls
  int64_t slab_bytes, page_bytes;
  int64_t T;
  const int64_t* seq_tokens;      // ragged batch: per-sequence token counts (device), or null
  int32_t n_pages, last_valid;    // pages holding tokens; tokens in the last one
  int32_t nq;                     // queries per sequence: rows b * nq + i (1: one query)
  int32_t splits;
  int32_t kv_heads, q_heads;
  int32_t q_bf16;
  float qscale;                   // sm_scale * log2(e)
  PageMap pm;                     // pages of the layer (slab or paged)
};

// Page layout of cache type FMT (key codes of KB bits for SYM_TOKEN, value
// codes of VB bits for the per-token value types), as include/kvq.h lays it out.
template <int FMT, int D, int KB, int VB>
struct PagedGeom {
  static constexpr bool BF16 = FMT == KVQ_BF16_CACHE;
  static constexpr bool SYMK = FMT == KVQ_SYM_TOKEN;
  static constexpr int KROW = BF16 ? 2 * D : SYMK ? D * KB / 8 : D;   // bytes per key token row
  static constexpr int KCODES = 32 * KROW;           // the K rows (chunk-permuted in LDS)
  static constexpr int OFF_KS = KCODES;              // SYM_TOKEN: fp32 key scale per token
  static constexpr int OFF_VC = SYMK ? OFF_KS + 128 : KCODES;   // V cols
  static constexpr int VCODES = BF16 ? 64 * D : (FMT == KVQ_FP8_E4M3 || FMT == KVQ_FP8_E5M2) ? 32 * D
                                                                                               : 32 * D * VB / 8;
  static constexpr int OFF_VS = OFF_VC + VCODES;     // per-token value scale (code values)
  static constexpr int OFF_VZ = OFF_VS + 128;        // per-token value offset (FP8K_KIVIV)
  // staged in LDS per page: bfloat16 keys only; FP8 keys and values; per-token
  // codes with their scales (and offsets)
  static constexpr int BYTES = BF16 ? KCODES : (FMT == KVQ_FP8_E4M3 || FMT == KVQ_FP8_E5M2) ? OFF_VS
                             : FMT == KVQ_FP8K_KIVIV ? OFF_VZ + 128 : OFF_VS + 128;
  static constexpr int DMA = (BYTES + 1023) / 1024;  // 16-byte-per-lane copies (the last may be partial)
  static constexpr int NBUF = 2;
  static constexpr int WAVE_LDS = NBUF * BYTES;
  static_assert(BYTES % 16 == 0, "whole 16-byte chunks");
};

// Two FP8 bytes (low or high half of w; E4M3, or E5M2 when E5) -> packed
// f16 / bf16, exact (both formats lie inside the f16 and bf16 ranges).
template <bool E5, bool HI>
__device__ __forceinline__ uint32_t fp8x2_f16(uint32_t w) {
  if constexpr (E5) return bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  else return bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
template <bool E5, bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  if constexpr (E5) return bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
  else return bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// FMT: KVQ_FP8_E4M3, KVQ_FP8_E5M2 or KVQ_BF16_CACHE; or a cache whose
// values are codes with a scale per token: KVQ_SYM_TOKEN (keys too: KB-bit
// codes with a scale per token), KVQ_FP8K_SYMV and KVQ_FP8K_KIVIV (E4M3 keys
// with the KV head's key scale; VB-bit values, symmetric or with a
// per-token offset). The E5M2 key scale is applied to the scores after the
// product instead of to q: with the scales that E5M2's range calls for
// (max |x| / 57344), q * ks would fall among the f16 subnormals.
// Per-token codes (2, 4 or 8 bits) convert exactly to f16 / bf16 as unsigned
// fields; a two's-complement field with its top bit flipped is the code plus
// 2^(b-1), so for symmetric codes
//   key:   q . (s_t k_t)  = s_t (q . u_t - 2^(KB-1) sum_c q_c)
//   value: sum_t p_t s_t v_t = sum_t (p_t s_t) u_t - sum_t p_t s_t 2^(VB-1)
// (u the flipped field), the value term being the per-token offset
// z_t = -2^(VB-1) s_t that KIVI values carry explicitly. The unsigned code
// converts give the channel (token) order {0,2,1,3,4,6,5,7} within each 8,
// which the query (weight) operand follows (8-bit codes keep their order).
// QN = 2 (GQA 4): two consecutive queries of a sequence per block,
// the second one's high and remainder columns and weight rows in the halves
// of the products that one query at GQA 4 leaves idle; the pages up to the
// second query's token, each column masking after its own query's.
template <int FMT, int D, int HG, int KB = 8, int VB = 8, int QN = 1>
__global__ __launch_bounds__(kThreads, 2) void paged_mfma_kernel(Fp8Params p) {
  static_assert(2 * HG * QN <= 16, "high and remainder columns of the GQA group(s) fit one tile");
  static_assert(QN == 1 || (QN == 2 && HG == 4), "two queries per block: GQA 4");
  constexpr int GC = HG * QN;             // (query, head) pairs of the block
  constexpr bool BF16 = FMT == KVQ_BF16_CACHE;
  constexpr bool E5 = FMT == KVQ_FP8_E5M2;
  constexpr bool SYMK = FMT == KVQ_SYM_TOKEN;                    // key codes, a scale per token
  constexpr bool CODEV = SYMK || FMT == KVQ_FP8K_SYMV || FMT == KVQ_FP8K_KIVIV;   // value codes
  constexpr bool ASYMV = FMT == KVQ_FP8K_KIVIV;                  // value offset per token
  static_assert(!SYMK || KB == 2 || KB == 4 || KB == 8, "2-, 4- or 8-bit key codes");
  static_assert(!CODEV || VB == 2 || VB == 4 || VB == 8, "2-, 4- or 8-bit value codes");
  constexpr bool PERMK = SYMK && KB < 8;    // key channels in the order {0,2,1,3,4,6,5,7}
  constexpr bool PERMV = CODEV && VB < 8;   // value tokens in that order
  using PG = PagedGeom<FMT, D, KB, VB>;
  constexpr int KS = D / 32;             // k-steps of the key product
  constexpr int NT = D / 16;             // channel tiles of the value product
  constexpr int CPG = D / 4;             // key channels per lane group (contiguous bytes)
  constexpr int RED = kWaves * GC * (D + 2) * 4;
  constexpr int ARENA = kWaves * PG::WAVE_LDS > RED ? kWaves * PG::WAVE_LDS : RED;

  __shared__ __attribute__((aligned(16))) float qs[GC][D];
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];
  __shared__ int last_block;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int j = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int rows_b = p.nq / QN;                    // grid rows per sequence
  const int b = blockIdx.z / rows_b, qi = (blockIdx.z - b * rows_b) * QN;   // sequence, its (first) query
  const int row = b * p.nq + qi;                   // query row b * nq + qi (of q, out, partials)
  // lane column j: query j / (2HG) of the block, high part when j % (2HG) < HG
  const bool col_hi = (j % (2 * HG)) < HG;
  const bool col_live = QN == 1 ? j < HG : col_hi;
  const int unit = b * p.kv_heads + h;             // one arrival counter for every row of b
  uint8_t* wbuf = arena + wave * PG::WAVE_LDS;
  const float ks_h = E5 ? p.k_scale[h] : 1.0f;   // applied to the scores (E5M2)

  // pages of this block, every kWaves-th one per wave
  // pages this sequence holds (a ragged batch: its own fill level), cut at
  // the query's own token when there are several (query qi of nq sits at
  // position fill - nq + qi)
  // (QN = 2: the pages up to the second query's token; the first query's
  // columns see one token less of the last page, possibly none)
  int32_t n_pages = p.n_pages, last_valid = p.last_valid;
  if (p.seq_tokens || p.nq > 1) {
    const int64_t Tb = seq_len(p.seq_tokens, b, p.T) - (p.nq - 1 - qi) + (QN - 1);
    n_pages = static_cast<int32_t>((Tb + kPage - 1) / kPage);
    last_valid = static_cast<int32_t>(Tb - static_cast<int64_t>(n_pages - 1) * kPage);
  }
  // the cache's open last page (fewer than 32 tokens) keeps FP8 values in
  // token rows (-1: every page is full)
  int open_page = -1;
  if constexpr (FMT == KVQ_FP8_E4M3 || FMT == KVQ_FP8_E5M2) {
    const int64_t fill = seq_len(p.seq_tokens, b, p.T);
    if (fill % kPage != 0) open_page = static_cast<int>(fill / kPage);
  }
  const int pg0 = static_cast<int>(static_cast<int64_t>(split) * n_pages / p.splits);
  const int pg1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_pages / p.splits);
  const int n_mine = pg0 + wave < pg1 ? (pg1 - pg0 - wave + kWaves - 1) / kWaves : 0;

  auto issue_page = [&](int k) {
    const uint8_t* src = p.pm.page(b, h, pg0 + wave + kWaves * k);
    const uint32_t dst = lds_addr(wbuf + (k % PG::NBUF) * PG::BYTES);
#pragma unroll
    for (int i = 0; i < PG::DMA; ++i) {
      const int off = i * 1024 + lane * 16;   // key rows: chunk permutation (see kswz)
      const int from = off < PG::KCODES ? krow_off<PG::KROW / 16>(off / PG::KROW, off % PG::KROW) : off;
      if (i + 1 < PG::DMA || off < PG::BYTES) dma16(src + from, dst + i * 1024);
    }
  };
  // bf16 values: lane (j, g) loads tokens 8g..8g+7 of channel 16 nt + j (16 bytes)
  auto load_values = [&](int k, uint4* vr) {
    const uint8_t* src = p.pm.page(b, h, pg0 + wave + kWaves * k) + PG::OFF_VC + 16 * g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      vr[nt] = *reinterpret_cast<const uint4*>(src + (16 * nt + j) * (kPage * 2));
  };
  uint4 va[BF16 ? NT : 1], vb[BF16 ? NT : 1];
  if (n_mine > 0) {   // in flight while the query is staged
    if constexpr (BF16) load_values(0, va);
    issue_page(0);
  }

  // ---- query group: q * sm_scale * log2(e) * ks_h ----------------------------
  {
    const float mult = (BF16 || E5 || SYMK) ? p.qscale : p.qscale * p.k_scale[h];
    for (int i = tid; i < GC * D; i += kThreads) {
      const int qq = i / (HG * D);   // the block's query qq: row + qq
      const int64_t q0 = (static_cast<int64_t>(row + qq) * p.q_heads + h * HG) * D + (i - qq * HG * D);
      const float x = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p.q)[q0])
                               : reinterpret_cast<const float*>(p.q)[q0];
      (&qs[0][0])[i] = x * mult;
    }
  }
  __syncthreads();
  // B operand of the key product for this lane: column j is head j % HG's
  // high part (j < HG), its remainder (HG <= j < 2HG) or zero.
  // (f16 parts against the E4M3 keys, bf16 parts against bf16 keys)
  using BQ = std::conditional_t<BF16, bf16x8, half8>;
  BQ bq[KS];
  // f16 range of the key operand: a query folded with a large key scale can
  // exceed 65504, where the f16 high part would saturate; then the wave takes
  // q' 2^-esc into the product and multiplies its scores by 2^esc (exact)
  int esc = 0;
  if constexpr (!BF16) {
    const int hh = (j / (2 * HG)) * HG + j % HG;   // pair of column j (QN = 1: head j % HG)
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) amax = fmaxf(amax, fabsf(qs[QN == 1 ? j % HG : hh][g * CPG + i]));
    if (__builtin_amdgcn_ballot_w64(amax > 65504.f) != 0) {
      amax = wave_max(amax);
      int ex;
      frexpf(amax, &ex);   // amax < 2^ex
      esc = __builtin_amdgcn_readfirstlane(ex - 15);
    }
  }
  // SYM_TOKEN keys: 2^(KB-1) times the sum of head j % HG's scaled query
  float kbias = 0.f;
  if constexpr (SYMK) {
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < CPG; ++i) sq += qs[QN == 1 ? j % HG : (j / (2 * HG)) * HG + j % HG][g * CPG + i];
    sq += xor16(sq);
    sq += xor32(sq);
    kbias = sq * static_cast<float>(1 << (KB - 1));
  }
  {
    const int hh = QN == 1 ? j % HG : (j / (2 * HG)) * HG + j % HG;
    const int part = QN == 1 ? j / HG : (j % (2 * HG)) / HG;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // pair i: channels (2i, 2i+1), or for key codes the converts' order
        // (0,2), (1,3), (4,6), (5,7)
        const int c0 = PERMK ? (i & 2) * 2 + (i & 1) : 2 * i, c1 = PERMK ? c0 + 2 : 2 * i + 1;
        const float a = ldexpf(qs[hh][g * CPG + 8 * ks + c0], -esc);
        const float c = ldexpf(qs[hh][g * CPG + 8 * ks + c1], -esc);
        uint32_t hi, lo;
        if constexpr (BF16) split_bf16(a, c, hi, lo);
        else split_f16(a, c, hi, lo);
        w4[i] = part == 0 ? hi : (part == 1 ? lo : 0u);
      }
      bq[ks] = __builtin_bit_cast(BQ, uint4{w4[0], w4[1], w4[2], w4[3]});
    }
  }

  // ---- per-wave online softmax -----------------------------------------------
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_lane = -INFINITY, l_lane = 0.f, z_lane = 0.f;

  // n_valid: tokens of the page the block's (last) query sees; n_valid0: the
  // first query's (QN = 2), for its columns
  auto process_page = [&](const uint8_t* pg, int n_valid, int n_valid0, const uint4* vr, bool vrows) {
    (void)vrows;   // bfloat16 caches: value columns on every page
    // scores; tile mt row rho = token 8(rho/4) + 4mt + rho%4
    float s[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int row = 8 * (j >> 2) + 4 * mt + (j & 3);
      floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (BF16) {
          const uint4 w = *reinterpret_cast<const uint4*>(
              pg + krow_off<PG::KROW / 16>(row, 2 * (g * CPG + 8 * ks)));
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), bq[ks], c, 0, 0, 0);
        } else if constexpr (SYMK && KB == 8) {   // bytes with the top bit flipped, as f16 integers
          const uint2 w = *reinterpret_cast<const uint2*>(pg + krow_off<PG::KROW / 16>(row, g * CPG + 8 * ks));
          const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u;
          const half8 a = cat4h(bits32(__builtin_amdgcn_cvt_pkrtz(float(x0 & 255u), float((x0 >> 8) & 255u))),
                                bits32(__builtin_amdgcn_cvt_pkrtz(float((x0 >> 16) & 255u), float(x0 >> 24))),
                                bits32(__builtin_amdgcn_cvt_pkrtz(float(x1 & 255u), float((x1 >> 8) & 255u))),
                                bits32(__builtin_amdgcn_cvt_pkrtz(float((x1 >> 16) & 255u), float(x1 >> 24))));
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[ks], c, 0, 0, 0);
        } else if constexpr (SYMK && KB == 4) {   // one word: the 8 channels of this k-step
          const uint32_t w = *reinterpret_cast<const uint32_t*>(
                                 pg + krow_off<PG::KROW / 16>(row, (g * CPG + 8 * ks) / 2)) ^ 0x88888888u;
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes4_frag(w), bq[ks], c, 0, 0, 0);
        } else if constexpr (SYMK) {   // one word: the 16 channels of k-steps ks, ks + 1
          if (ks % 2 == 0) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(
                                   pg + krow_off<PG::KROW / 16>(row, (g * CPG + 8 * ks) / 4)) ^ 0xAAAAAAAAu;
            half8 a0, a1;
            codes2_frags(w, a0, a1);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bq[ks], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bq[ks + 1], c, 0, 0, 0);
          }
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(pg + krow_off<D / 16>(row, g * CPG + 8 * ks));
          const half8 a = cat4h(fp8x2_f16<E5, false>(w.x), fp8x2_f16<E5, true>(w.x),
                                fp8x2_f16<E5, false>(w.y), fp8x2_f16<E5, true>(w.y));
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[ks], c, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * mt + r] = c[r] + row_shl<HG>(c[r]);
    }
    if constexpr (E5) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] *= ks_h;
    }
    if (esc != 0) {   // wave-uniform, rare: undo the range scaling of q'
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = ldexpf(s[i], esc);
    }
    if constexpr (SYMK) {   // s_t (q . u_t - 2^(KB-1) sum q) for tokens 8g..8g+7
      const float4 k0 = *reinterpret_cast<const float4*>(pg + PG::OFF_KS + 32 * g);
      const float4 k1 = *reinterpret_cast<const float4*>(pg + PG::OFF_KS + 32 * g + 16);
      const float kst[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = kst[i] * (s[i] - kbias);
    }
    const int nv_col = (QN == 2 && j < 2 * HG) ? n_valid0 : n_valid;   // this column's query
    if (nv_col < kPage) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = 8 * g + i < nv_col ? s[i] : -INFINITY;
    }
    // online softmax: running max per head (lanes j < HG), weights 2^(s - m)
    // (whether a head's max grows is decided by each lane's own maximum; the
    // maximum over the head's four lane groups is only formed when one does)
    float pmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) pmax = fmaxf(pmax, s[i]);
    if (__builtin_amdgcn_ballot_w64(col_live && (pmax > m_lane)) != 0) {
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      const float m_new = fmaxf(m_lane, pmax);
      // (QN = 2: a column whose max stays -inf while the other query's move
      // keeps its sums; 2^(-inf - -inf) would be NaN)
      const float alpha = (QN == 2 && m_new == m_lane) ? 1.0f : fast_exp2(m_lane - m_new);
      l_lane *= alpha;
      z_lane *= alpha;
      m_lane = m_new;
      auto alpha_of = [&](int hh) {   // head hh's factor, read from lane hh
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), hh));
      };
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float a = alpha_of(r % HG);
        // HG = 8: rows 4g + r are head r (g even) or head 4 + r (g odd); a
        // choice between two values (an index into an array of the factors
        // would be compiled into a stack load)
        if constexpr (HG == 8) {
          const float a_odd = alpha_of(4 + r);
          a = (g & 1) ? a_odd : a;
        }
        // QN = 2: rows 4g + r of lane groups 2, 3 belong to the second query,
        // whose head r is column 2HG + r
        if constexpr (QN == 2) {
          const float a_q1 = alpha_of(2 * HG + r);
          a = g >= 2 ? a_q1 : a;
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= a;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = fast_exp2(s[i] - m_lane);
    if constexpr (QN == 2) {
      // a column that has seen no token yet (max -inf) gets weight 0 for its
      // absent tokens (2^(-inf - -inf) is not 0)
      if (nv_col < kPage) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = 8 * g + i < nv_col ? s[i] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) l_lane += s[i];
    // per-token value codes: P' = p s_t (tokens 8g..8g+7), sum of p z_t; an
    // absent token's scale and offset are taken as 0 (its bytes are undefined)
    if constexpr (CODEV) {
      const float4 v0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + 32 * g);
      const float4 v1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + 32 * g + 16);
      float vsv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float vzv[8];
      if constexpr (ASYMV) {
        const float4 z0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + 32 * g);
        const float4 z1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + 32 * g + 16);
        vzv[0] = z0.x; vzv[1] = z0.y; vzv[2] = z0.z; vzv[3] = z0.w;
        vzv[4] = z1.x; vzv[5] = z1.y; vzv[6] = z1.z; vzv[7] = z1.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vzv[i] = -static_cast<float>(1 << (VB - 1)) * vsv[i];
      }
      if (n_valid < kPage) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool ok = 8 * g + i < n_valid;
          vsv[i] = ok ? vsv[i] : 0.f;
          vzv[i] = ok ? vzv[i] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) z_lane = fmaf(s[i], vzv[i], z_lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] *= vsv[i];
    }
    // P rows: j < HG high part of head j, HG <= j < 2HG remainder of head j-HG
    // (value codes: tokens in the converts' order {0,2,1,3,4,6,5,7})
    uint32_t ph[4], pl[4], pa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t0 = PERMV ? (i & 2) * 2 + (i & 1) : 2 * i, t1 = PERMV ? t0 + 2 : 2 * i + 1;
      split_bf16(s[t0], s[t1], ph[i], pl[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = shr_keep<HG>(ph[i], pl[i]);
      if constexpr (QN == 2) pa[i] = col_hi ? ph[i] : pa[i];   // the second query's high rows keep theirs
    }
    const bf16x8 ap = __builtin_bit_cast(bf16x8, uint4{pa[0], pa[1], pa[2], pa[3]});
    if constexpr (BF16) {
      // values of tokens 8g..8g+7 of channel 16 nt + j (registers); absent
      // tokens -> 0 (word w holds tokens 8g+2w, 8g+2w+1)
      uint32_t mw[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
      if (n_valid < kPage) {
        const int k = min(max(n_valid - 8 * g, 0), 8);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mw[w] = 2 * w + 2 <= k ? 0xFFFFFFFFu : (2 * w + 1 == k ? 0x0000FFFFu : 0u);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint4 bw = uint4{vr[nt].x & mw[0], vr[nt].y & mw[1], vr[nt].z & mw[2], vr[nt].w & mw[3]};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt],
                                                           0, 0, 0);
      }
    } else if constexpr (CODEV) {
      (void)vr;
      // value codes of tokens 8g..8g+7 of channel 16 nt + j (the column's
      // bits [8 VB g, 8 VB (g + 1))); symmetric codes with the top bit flipped
      constexpr int VROW = 32 * VB / 8;   // bytes per channel column
      constexpr uint32_t FLIP = ASYMV ? 0u : (VB == 8 ? 0x80808080u : VB == 4 ? 0x88888888u : 0xAAAAAAAAu);
      if constexpr (VB == 8) {   // bytes as bf16 integers (exact up to 256), tokens in order
        auto bf2 = [](uint32_t lo, uint32_t hi) {   // two small integers -> packed bf16 (exact)
          return (__float_as_uint(float(lo)) >> 16) | (__float_as_uint(float(hi)) & 0xFFFF0000u);
        };
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 w = *reinterpret_cast<const uint2*>(pg + PG::OFF_VC + (16 * nt + j) * VROW + 8 * g);
          const uint32_t x0 = w.x ^ FLIP, x1 = w.y ^ FLIP;
          const uint4 bw{bf2(x0 & 255u, (x0 >> 8) & 255u), bf2((x0 >> 16) & 255u, x0 >> 24),
                         bf2(x1 & 255u, (x1 >> 8) & 255u), bf2((x1 >> 16) & 255u, x1 >> 24)};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
        }
      } else if constexpr (VB == 4) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(pg + PG::OFF_VC + (16 * nt + j) * VROW + 4 * g) ^ FLIP;
          const uint32_t y0 = w & 0x0F0F0F0Fu, y1 = (w >> 4) & 0x0F0F0F0Fu;
          const uint4 bw{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, false)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, false)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, true)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, true))};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; nt += 2) {   // two channel tiles per word
          const uint8_t* col = pg + PG::OFF_VC + (16 * nt + j) * VROW + 2 * g;
          const uint32_t x = (uint32_t(*reinterpret_cast<const uint16_t*>(col)) |
                              (uint32_t(*reinterpret_cast<const uint16_t*>(col + 16 * VROW)) << 16)) ^ FLIP;
          const uint32_t y0 = x & 0x33333333u, y1 = (x >> 2) & 0x33333333u;
          const uint4 b0{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 0)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 0)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 1)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 1))};
          const uint4 b1{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 2)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 2)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 3)),
                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 3))};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, b0), acc[nt], 0, 0, 0);
          acc[nt + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, b1), acc[nt + 1], 0, 0, 0);
        }
      }
    } else {
      (void)vr;
      // value bytes of tokens 8g..8g+7 of channel 16 nt + j; absent tokens -> 0
      uint32_t m0 = 0xFFFFFFFFu, m1 = 0xFFFFFFFFu;
      if (n_valid < kPage) {
        const int k = min(max(n_valid - 8 * g, 0), 8);
        m0 = k >= 4 ? 0xFFFFFFFFu : (1u << (8 * k)) - 1u;
        m1 = k >= 8 ? 0xFFFFFFFFu : (k <= 4 ? 0u : (1u << (8 * (k - 4))) - 1u);
      }
      if (vrows) {   // wave-uniform, one page per row: tokens 8g..8g+7 from their rows
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint8_t* col = pg + PG::OFF_VC + 8 * g * D + 16 * nt + j;
          uint32_t x0 = 0u, x1 = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x0 |= uint32_t(col[i * D]) << (8 * i);
            x1 |= uint32_t(col[(4 + i) * D]) << (8 * i);
          }
          x0 &= m0;
          x1 &= m1;
          const uint4 bw = uint4{fp8x2_bf16<E5, false>(x0), fp8x2_bf16<E5, true>(x0),
                                 fp8x2_bf16<E5, false>(x1), fp8x2_bf16<E5, true>(x1)};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt],
                                                             0, 0, 0);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 w = *reinterpret_cast<const uint2*>(pg + PG::OFF_VC + (16 * nt + j) * kPage + 8 * g);
          const uint32_t x0 = w.x & m0, x1 = w.y & m1;
          const uint4 bw = uint4{fp8x2_bf16<E5, false>(x0), fp8x2_bf16<E5, true>(x0),
                                 fp8x2_bf16<E5, false>(x1), fp8x2_bf16<E5, true>(x1)};
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt],
                                                             0, 0, 0);
        }
      }
    }
  };

  // ---- pages: DMA pipeline, one page ahead ----------------------------------
  // (bf16: the value registers of page k+1 are requested before the key rows,
  // so waiting for at most NT + DMA requests leaves page k's complete)
  auto step = [&](int k, const uint4* cur, uint4* nxt) {
    wait_lds();   // the buffer about to be refilled has been read
    __builtin_amdgcn_wave_barrier();
    const bool next = k + 1 < n_mine;
    if (next) {
      if constexpr (BF16) load_values(k + 1, nxt);
      issue_page(k + 1);
      wait_vm<(BF16 ? NT : 0) + PG::DMA>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_wave_barrier();
    const int page = pg0 + wave + kWaves * k;
    const bool last = page == n_pages - 1;
    process_page(wbuf + (k % PG::NBUF) * PG::BYTES, last ? last_valid : kPage,
                 last ? last_valid - (QN - 1) : kPage, cur, page == open_page);
  };
#pragma unroll 1
  for (int k = 0; k < n_mine; k += 2) {
    step(k, va, vb);
    if (k + 1 < n_mine) step(k + 1, vb, va);
  }
  wait_lds();

  // ---- wave epilogue -----------------------------------------------------------
  // per (query, head) pair vh: its column (vh / HG) 2HG + vh % HG
  float lsum[GC], mh[GC], zsum[GC];
  {
    float l_ = l_lane, z_ = z_lane;
    l_ += xor16(l_);
    l_ += xor32(l_);
    if constexpr (CODEV) {
      z_ += xor16(z_);
      z_ += xor32(z_);
    }
#pragma unroll
    for (int vh = 0; vh < GC; ++vh) {
      const int col = (vh / HG) * 2 * HG + vh % HG;
      lsum[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_), col));
      mh[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_lane), col));
      zsum[vh] = CODEV ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z_), col)) : 0.f;
    }
  }
  __syncthreads();   // every wave is done with its page buffers (the arena)
  float* red = reinterpret_cast<float*>(arena);   // [wave][GC][D + 2]: m, l, o
  auto R = [&](int w, int vh) { return red + (w * GC + vh) * (D + 2); };
  // acc rows 4g+r: row < HG is head row (high), HG <= row < 2HG head row-HG
  // (remainder); with two queries rows 2HG.. repeat that for the second
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = acc[nt][r];
      if constexpr (HG == 1) {
        x = r == 0 ? acc[nt][0] + acc[nt][1] : 0.f;
      } else if constexpr (HG == 2) {
        x = r < 2 ? acc[nt][r] + acc[nt][r + 2] : 0.f;
      } else if constexpr (HG == 4) {
        x += xor16(x);
      } else {
        x += xor32(x);
      }
      v[r] = x;
    }
    const int c = 16 * nt + j;
    if ((4 * g) % (2 * HG) < HG && 4 * g < 2 * GC) {   // lane groups holding the high rows
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hh = (4 * g) % (2 * HG) + r;
        const int vh = (4 * g / (2 * HG)) * HG + hh;
        float zz = 0.f;   // sum of p z (value codes) of pair vh
#pragma unroll
        for (int k = 0; k < GC; ++k) zz = vh == k ? zsum[k] : zz;
        if (hh < HG) R(wave, vh)[2 + c] = v[r] + zz;
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int vh = 0; vh < GC; ++vh) {
      R(wave, vh)[0] = mh[vh];
      R(wave, vh)[1] = lsum[vh];
    }
  }
  __syncthreads();
  // several blocks per (sequence, KV head): count this block's arrival first;
  // the round trip overlaps the combination of the waves below
  int arrived = 0;
  if (p.splits > 1 && tid == 0) arrived = count_arrival(&p.counters[unit]);

  // ---- combine the waves: this thread's elements i = tid + e * kThreads ----
  const float vs_h = (BF16 || CODEV) ? 1.0f : p.v_scale[h];
  constexpr int PER = (GC * D + kThreads - 1) / kThreads;
  float own_m[PER], own_l[PER], own_o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = tid + e * kThreads;
    own_m[e] = -INFINITY;
    own_l[e] = 0.f;
    own_o[e] = 0.f;
    if (i < GC * D) {
      const int vh = i / D, c = i % D;   // pair vh: query vh / HG of the block, head vh % HG
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, R(w, vh)[0]);
      float so = 0.f, sl = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float ew = exp2_rel(R(w, vh)[0], M);   // idle wave (or block): 0
        so = fmaf(ew, R(w, vh)[2 + c], so);
        sl = fmaf(ew, R(w, vh)[1], sl);
      }
      so *= vs_h;
      if (p.splits == 1)
        p.out[(static_cast<int64_t>(row + vh / HG) * p.q_heads + h * HG + vh % HG) * D + c] = so / sl;
      own_m[e] = M;
      own_l[e] = sl;
      own_o[e] = so;
    }
  }
  if (p.splits == 1) return;

  // ---- the last of the (nq / QN) * splits blocks of (b, h) to arrive merges --
  if (tid == 0) last_block = arrived == (p.nq / QN) * p.splits - 1;
  __syncthreads();
  if constexpr (QN == 1) {
    float* part_rh = p.partials + (static_cast<int64_t>(row) * p.q_heads + h * HG) * p.splits * (D + 2);
    if (!last_block) {
      store_partial<D, HG, kThreads>(part_rh, p.splits, split, own_m, own_l, own_o, tid);
      return;
    }
    merge_partials<D, HG, kThreads>(p.partials, p.out, &p.counters[unit], p.q_heads, p.splits, p.nq, b, h,
                                    row, split, own_m, own_l, own_o, tid);
  } else {
    // every block stores the partials of its rows; the last one merges them
    // all from memory (row -1: none from registers)
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * kThreads;
      if (i < GC * D) {
        const int vh = i / D, c = i % D;
        float* part = p.partials +
                      ((static_cast<int64_t>(row + vh / HG) * p.q_heads + h * HG + vh % HG) * p.splits + split) *
                          (D + 2);
        put_partial(part + 2 + c, own_o[e]);
        if (c == 0) {
          put_partial(part, own_m[e]);
          put_partial(part + 1, own_l[e]);
        }
      }
    }
    if (!last_block) return;
    merge_partials<D, HG, kThreads>(p.partials, p.out, &p.counters[unit], p.q_heads, p.splits, p.nq, b, h, -1,
                                    split, own_m, own_l, own_o, tid);
  }
}

// batch: grid rows (sequences x queries / qn); qn 2: two queries per block (GQA 4)
template <int FMT, int D, int KB, int VB>
hipError_t by_hg(const Fp8Params& p, int hg, int batch, hipStream_t st, int qn = 1) {
  dim3 grid(p.splits, p.kv_heads, batch);
  switch (hg) {
    case 1: hipLaunchKernelGGL((paged_mfma_kernel<FMT, D, 1, KB, VB>), grid, dim3(kThreads), 0, st, p); break;
    case 2: hipLaunchKernelGGL((paged_mfma_kernel<FMT, D, 2, KB, VB>), grid, dim3(kThreads), 0, st, p); break;
    case 4:
      if (qn == 2) {
        hipLaunchKernelGGL((paged_mfma_kernel<FMT, D, 4, KB, VB, 2>), grid, dim3(kThreads), 0, st, p);
        break;
      }
      hipLaunchKernelGGL((paged_mfma_kernel<FMT, D, 4, KB, VB>), grid, dim3(kThreads), 0, st, p);
      break;
    default: hipLaunchKernelGGL((paged_mfma_kernel<FMT, D, 8, KB, VB>), grid, dim3(kThreads), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int FMT, int KB = 8, int VB = 8>
hipError_t by_d(const Fp8Params& p, int d, int hg, int batch, hipStream_t st, int qn = 1) {
  switch (d) {
    case 32:
      if constexpr (!(FMT == KVQ_SYM_TOKEN && KB == 2)) return by_hg<FMT, 32, KB, VB>(p, hg, batch, st, qn);
      return hipErrorInvalidValue;   // not routed here (fp8_mfma_path)
    case 64: return by_hg<FMT, 64, KB, VB>(p, hg, batch, st, qn);
    case 128: return by_hg<FMT, 128, KB, VB>(p, hg, batch, st, qn);
    default: return by_hg<FMT, 256, KB, VB>(p, hg, batch, st, qn);
  }
}

}  // namespace

// FP8 (either format) and bf16 caches, and caches of per-token codes at 2, 4
// or 8 bits (symmetric keys and values; FP8 keys with symmetric or KIVI values)
// take the matrix-core paged kernel (head_dim >= 32, no rotary embedding;
// at head_dim 32 a 2-bit symmetric key row is 8 bytes, less than the 16-byte
// chunk the page staging permutes, and stays on the generic kernel).
bool fp8_mfma_path(const Geometry& g) {
  if (g.rope != 0.0 || g.d < 32) return false;
  if (g.d == 32 && g.scheme == KVQ_SYM_TOKEN && g.bits == 2) return false;
  if (is_fp8(g.scheme) || g.scheme == KVQ_BF16_CACHE) return true;
  if (g.scheme == KVQ_SYM_TOKEN) return g.bits == 2 || g.bits == 4 || g.bits == 8;
  if (is_fp8_keys_mixed(g.scheme)) return g.vbits == 2 || g.vbits == 4 || g.vbits == 8;
  return false;
}

int32_t fp8_mfma_splits(const Geometry& g, int64_t tokens, int32_t requested) {
  const int64_t pages = (tokens + kPage - 1) / kPage;
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    // about one resident round of blocks (two per CU on 256 CUs), >= 8 pages each
    const int64_t units = static_cast<int64_t>(g.batch) * g.kv_heads;
    s = (512 + units - 1) / units;
    const int64_t cap = (pages + 7) / 8;
    if (s > cap) s = cap;
  }
  if (s > pages) s = pages;
  return static_cast<int32_t>(s < 1 ? 1 : s);
}

hipError_t launch_fp8_mfma(const DecodeArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const int32_t nq = a.nq > 1 ? a.nq : 1;
  // several queries per sequence: batch * nq rows, and the split count
  // planned for that many (never more than the one-query plan, whose
  // workspace nq copies of hold the partials)
  // two queries per block: GQA 4, an even number of queries
  const int qn = (g.hg == 4 && nq >= 2 && nq % 2 == 0) ? 2 : 1;
  Geometry rows = g;
  rows.batch = g.batch * nq / qn;
  Fp8Params p{};
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
  p.T = a.tokens;
  p.seq_tokens = a.seq_tokens;
  p.n_pages = static_cast<int32_t>((a.tokens + kPage - 1) / kPage);
  p.last_valid = static_cast<int32_t>(a.tokens - static_cast<int64_t>(p.n_pages - 1) * kPage);
  p.nq = nq;
  p.splits = fp8_mfma_splits(rows, a.tokens, a.requested_splits);
  p.kv_heads = g.kv_heads;
  p.q_heads = g.q_heads;
  p.q_bf16 = a.q_dtype == KVQ_BF16;
  p.qscale = a.sm_scale * kLog2e;
  const int rows_n = g.batch * nq / qn;
  switch (g.scheme) {
    case KVQ_BF16_CACHE: return by_d<KVQ_BF16_CACHE>(p, g.d, g.hg, rows_n, st, qn);
    case KVQ_FP8_E5M2: return by_d<KVQ_FP8_E5M2>(p, g.d, g.hg, rows_n, st, qn);
    case KVQ_SYM_TOKEN:
      return g.bits == 2   ? by_d<KVQ_SYM_TOKEN, 2, 2>(p, g.d, g.hg, rows_n, st, qn)
             : g.bits == 4 ? by_d<KVQ_SYM_TOKEN, 4, 4>(p, g.d, g.hg, rows_n, st, qn)
                           : by_d<KVQ_SYM_TOKEN, 8, 8>(p, g.d, g.hg, rows_n, st, qn);
    case KVQ_FP8K_SYMV:
      return g.vbits == 2   ? by_d<KVQ_FP8K_SYMV, 8, 2>(p, g.d, g.hg, rows_n, st, qn)
             : g.vbits == 4 ? by_d<KVQ_FP8K_SYMV, 8, 4>(p, g.d, g.hg, rows_n, st, qn)
                            : by_d<KVQ_FP8K_SYMV, 8, 8>(p, g.d, g.hg, rows_n, st, qn);
    case KVQ_FP8K_KIVIV:
      return g.vbits == 2   ? by_d<KVQ_FP8K_KIVIV, 8, 2>(p, g.d, g.hg, rows_n, st, qn)
             : g.vbits == 4 ? by_d<KVQ_FP8K_KIVIV, 8, 4>(p, g.d, g.hg, rows_n, st, qn)
                            : by_d<KVQ_FP8K_KIVIV, 8, 8>(p, g.d, g.hg, rows_n, st, qn);
    default: return by_d<KVQ_FP8_E4M3>(p, g.d, g.hg, rows_n, st, qn);
  }
}

}  // namespace kvq
