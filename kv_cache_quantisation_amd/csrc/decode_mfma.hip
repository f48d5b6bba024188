// Decode attention over a KIVI 2/4-bit cache on the matrix cores (gfx950).
//
// Same result as the generic kernel -- softmax(sm_scale q.K^) . V^ over the
// dequantised cache ("Quantizing the KV cache", going deeper) -- organised for
// v_mfma_f32_16x16x32_{f16,bf16}. For one 32-token page of one (sequence, KV
// head):
//
//   keys:   S^T[t][h] = sum_c code_tc q'_hc + b_h,  q'_hc = q_hc s_c,
//           b_h = sum_c q_hc z_c       (per-channel scale and offset folded in)
//           A = key codes [16 tokens x 32 channels] as exact f16 integers,
//           B = q'^T [32 channels x 16 columns]: columns 0..HG-1 hold the f16
//           "hi" part of each GQA head's q', columns HG..2HG-1 the f16 "lo"
//           remainder q' - hi (together ~22 bits); the column groups are added
//           after the product.
//   values: O[h][c] += sum_t P'_ht code_tc,  P'_ht = p_ht s_t, plus
//           sum_t p_ht z_t added to every channel at the end.
//           v_mfma_f32_16x16x32_bf16: A = P' [16 rows x 32 tokens] (rows
//           0..HG-1 the bf16 nearest value, HG..2HG-1 the bf16 remainder: 16
//           bits at any magnitude, so tiny weights keep their relative
//           precision), B = value codes [32 tokens x 16 channels] as exact
//           bf16 integers.
//
// The unquantised residual tokens (bf16) take the same path 8 tokens at a
// time (one half of a 16-row tile): A = key rows as stored, B = q split into three bf16 parts (hi, mid,
// lo columns); P (split hi/lo in bf16) times the value rows, gathered per
// channel from LDS. They update the same softmax state and accumulators.
//
// Operand layouts (wave64): lane l holds A[l%16][8(l/16)+i], B[8(l/16)+i][l%16]
// (i = 0..7) and C[4(l/16)+r][l%16] (r = 0..3). Computing S^T (tokens as rows,
// row r of key tile mt holding token 8(r/4) + 4mt + r%4) leaves lane (j, g) =
// (l%16, l/16) with head j's scores for tokens 8g..8g+7: the lane and token set
// the P.V A-operand needs, so P never moves between lanes, and for channel c
// those tokens are the 16 bits at byte 2g of its 2-bit column (32 bits at byte
// 4g of its 4-bit column; the rotary variant keeps token 16mt + r in row r and
// picks bytes g and 4+g of a 2-bit column). Codes become exact small integers
// with the scaled converts:
// a 2-bit code in an FP4 E2M1 nibble is code/2 (scale 2), a 4-bit code in an
// FP8 E4M3 byte is code * 2^-9 (scale 512), to f16 for keys and bf16 for
// values; the converts produce channels in the order {0,2,1,3,4,6,5,7} within
// each 8, and q' is laid out to match.
//
// Memory: each wave streams its pages HBM -> LDS with global_load_lds_dwordx4
// (16 bytes per lane, a whole page in 4-11 instructions), one page ahead of
// the one it computes, so fetches overlap arithmetic without holding
// registers; `s_waitcnt vmcnt` retires them in issue order.
//
// Online softmax per head in the log2 domain (q pre-scaled by sm_scale*log2 e);
// the accumulators are rescaled only when some head's running max grows. Each
// block writes a partial (m, l, o) per query head; the last block of a
// (sequence, KV head) to finish merges them (a single block writes the output).
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_merge.h"
#include "kvq_wave.h"

namespace kvq {
namespace {


constexpr int kWaves = 4;
constexpr int kRopeWaves = 4;      // waves per block of rope4_kernel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxSlack = 8.0f;  // log2 units a score may exceed the running max by

struct MfmaParams {
  const uint8_t* layer_base;
  const uint8_t* q;
  float* out;
  float* partials;
  int* counters;                  // one per (sequence, KV head), zero between calls
  int64_t slab_bytes, page_bytes, ring_base, ring_slots;
  int64_t T, q_tokens;            // cached tokens; tokens held in pages
  const int64_t* seq_tokens;      // ragged batch: per-sequence token counts (device), or null
  int32_t n_pages, n_steps;       // quantised pages; residual tokens in 8-token steps
  int32_t residual;               // R (the flush plan of a ragged sequence)
  int32_t nq;                     // queries per sequence: rows b * nq + i (1: one query)
  int32_t splits;                 // blocks per (sequence, KV head)
  int32_t kv_heads, q_heads;
  int32_t q_bf16;
  float qscale;
  double rope_theta;              // > 0: keys cached before the rotary embedding
  // one-token append fused into the decode (kivi_mfma_kernel): the token at
  // position new_tok (>= 0; -1: none) is read from k_new / v_new
  // [batch][kv_heads][D] for its residual step, and the wave that takes that
  // step stores it into its ring slot
  const uint8_t* k_new;
  const uint8_t* v_new;
  int64_t new_tok;
  PageMap pm;                     // pages and rings of the layer (slab or paged)
};

// KIVI page of KB-bit key codes and VB-bit value codes
template <int KB, int VB, int D>
struct PageGeom {
  static constexpr int CODES = 32 * D * KB / 8;     // the packed K rows
  static constexpr int VCODES = 32 * D * VB / 8;    // the packed V cols
  static constexpr int OFF_KS = CODES;
  static constexpr int OFF_KZ = OFF_KS + 4 * D;
  static constexpr int OFF_VC = OFF_KZ + 4 * D;
  static constexpr int OFF_VS = OFF_VC + VCODES;
  static constexpr int OFF_VZ = OFF_VS + 128;
  static constexpr int BYTES = OFF_VZ + 128;
  static constexpr int DMA = (BYTES + 1023) / 1024;  // 16-byte-per-lane copies per page
  static constexpr int NBUF = 2;                       // page buffers per wave
  static constexpr int RING = 2 * 8 * D * 2;          // 8 key + 8 value bf16 rows
  static constexpr int WAVE_LDS = NBUF * BYTES + RING;
};

// Page token held by row r of the 16-row key tile mt. The C layout of the key
// product gives lane group g rows 4g..4g+3 of each tile, so with this map lane
// group g ends with the scores of tokens 8g..8g+7: the contiguous run of a
// value column that the P.V operand of the same lanes needs.
// The rotary variant keeps token 16mt + r in row r (its residual steps rotate
// tile row j by j with the same per-lane table), so lane group g holds tokens
// 4g..4g+3 and 16+4g..16+4g+3.
template <bool ROPE>
__device__ __forceinline__ int tile_tok(int mt, int r) {
  return ROPE ? 16 * mt + r : 8 * (r >> 2) + 4 * mt + (r & 3);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float load_q(const uint8_t* base, int64_t idx, int bf16) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

// ---- end of every decode kernel of this file -------------------------------
// Combines the block's waves (their running max mh, sums of p and p z per
// (query, head) pair, and value accumulators acc: rows 4g + r, per query the
// high parts of its heads, then their remainders), writes the output rows
// (one split) or the block's partials, and in the last block of a (sequence,
// KV head) to finish merges every partial. QN: queries of the block, rows
// b * nq + qi + qq of q, out and the partials. DIRECT: acc rows 4g + r are
// the pairs 4g + r themselves (kivi_deq_kernel).
template <int D, int HG, int NW = kWaves, int QN = 1, bool DIRECT = false>
__device__ __forceinline__ void finish_unit(const MfmaParams& p, const floatx4* acc, const float* mh,
                                            const float* lsum, const float* zsum, uint8_t* arena,
                                            int& last_block, int b, int qi, int h, int split) {
  constexpr int NT = D / 16;
  constexpr int NTH = NW * 64;             // threads of the block
  constexpr int GC = HG * QN;              // (query, head) pairs
  static_assert(QN == 1 || HG == 4, "several queries per block: GQA 4");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int j = lane & 15, g = lane >> 4;
  const int unit = b * p.kv_heads + h;   // one arrival counter for every query row of b
  const int row = b * p.nq + qi;         // the block's (first) query row (q, out, partials)
  __syncthreads();   // every wave is done with its page buffers (the arena)
  float* red = reinterpret_cast<float*>(arena);   // [wave][GC][D + 2]: m, l, o
  auto R = [&](int w, int vh) { return red + (w * GC + vh) * (D + 2); };
  if constexpr (DIRECT) {   // acc rows 4g+r: pair 4g+r
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vh = 4 * g + r;
        float zz = 0.f;   // sum_t p z_t of pair vh goes to every channel
#pragma unroll
        for (int k = 0; k < GC; ++k) zz = vh == k ? zsum[k] : zz;
        if (vh < GC) R(wave, vh)[2 + 16 * nt + j] = acc[nt][r] + zz;
      }
  } else
  // acc rows 4g+r: row < HG is head row (hi), HG <= row < 2HG is head row-HG
  // (lo); with two queries rows 2HG.. repeat that for the second query
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
        x += xor16(x);          // rows 0-3 (g=0) + rows 4-7 (g=1); with QN = 2, 8-11 + 12-15
      } else {
        x += xor32(x);          // rows 0-7 (g=0,1) + rows 8-15 (g=2,3)
      }
      v[r] = x;
    }
    const int c = 16 * nt + j;
    if ((4 * g) % (2 * HG) < HG && 4 * g < 2 * GC) {   // lane groups holding the high rows
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vh = (4 * g / (2 * HG)) * HG + (4 * g) % (2 * HG) + r;
        float zz = 0.f;   // sum_t p z_t of pair vh goes to every channel
#pragma unroll
        for (int k = 0; k < GC; ++k) zz = vh == k ? zsum[k] : zz;
        if ((4 * g) % (2 * HG) + r < HG) R(wave, vh)[2 + c] = v[r] + zz;
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

  // ---- combine the waves: this thread's elements i = tid + e * NTH --------
  // (element i: pair vh = i / D -- query vh / HG, head vh % HG -- channel i % D)
  constexpr int PER = (GC * D + NTH - 1) / NTH;
  float own_m[PER], own_l[PER], own_o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = tid + e * NTH;
    own_m[e] = -INFINITY;
    own_l[e] = 0.f;
    own_o[e] = 0.f;
    if (i < GC * D) {
      const int vh = i / D, c = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, R(w, vh)[0]);
      float so = 0.f, sl = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float ew = exp2_rel(R(w, vh)[0], M);   // idle wave (or block): 0
        so = fmaf(ew, R(w, vh)[2 + c], so);
        sl = fmaf(ew, R(w, vh)[1], sl);
      }
      const int r_out = row + vh / HG, hh = vh % HG;
      if (p.splits == 1) p.out[(static_cast<int64_t>(r_out) * p.q_heads + h * HG + hh) * D + c] = so / sl;
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
      store_partial<D, HG, NTH>(part_rh, p.splits, split, own_m, own_l, own_o, tid);
      return;
    }
    merge_partials<D, HG, NTH>(p.partials, p.out, &p.counters[unit], p.q_heads, p.splits, p.nq, b, h, row,
                               split, own_m, own_l, own_o, tid);
  } else {
    // every block stores the partials of its rows (each row's [HG][splits]
    // block of slots, element i of pair vh at row + vh / HG); the last one
    // merges them all from memory
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * NTH;
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
    // (row -1: no row's state comes from registers; every slot is read and cleared)
    merge_partials<D, HG, NTH>(p.partials, p.out, &p.counters[unit], p.q_heads, p.splits, p.nq, b, h, -1,
                               split, own_m, own_l, own_o, tid);
  }
}

// Blocks of the four-wave kivi_mfma_kernel<bits, *, d, *, rope> resident per
// CU (bits = key bits; value codes are never wider than key codes): what its
// LDS (page buffers, fragments, query) and registers are sized for. The split
// plan fills one round of the 256 CUs with this many blocks each.
constexpr int kivi_blocks_per_cu(int bits, int d, bool rope) {
  if (rope) return 2;
  if (d >= 256) return bits == 2 ? 2 : 1;
  return 3;
}

// Waves per block of kivi_mfma_kernel<kb, vb, d, hg, rope>: eight for 2-bit
// value codes (2- or 4-bit keys) at d <= 128 and GQA groups up to 4 (run as
// one block per CU: half the blocks, and half the partials to merge, of
// four-wave blocks; 2-bit keys 19.8 vs 20.5 us, 4-bit keys 21.5-21.8 vs
// 23.0-23.2 us at batch 16, context 4096), four otherwise. Eight-wave 2-bit
// blocks still fit two per CU (71.7 KB of LDS, <= 128 VGPRs), which
// kivi_blocks_per_cu(2, d, false) = 3 would only tighten, so their launch
// bound asks for two (4-bit keys: 88 KB of LDS, one per CU).
constexpr int kivi_waves(int kb, int vb, int d, int hg, bool rope) {
  return ((kb == 2 || kb == 4) && vb == 2 && d <= 128 && hg <= 4 && !rope) ? 8 : 4;
}

// KB, VB: bits of the key and of the value codes. QN: queries of a sequence
// per block (2: two consecutive queries share every page; their high and
// remainder columns fill the 16 columns of the key product and the 16 rows
// of the value product, which one query at GQA 4 fills half of)
template <int KB, int VB, int D, int HG, bool ROPE, int QN = 1>
__global__ __launch_bounds__(64 * kivi_waves(KB, VB, D, HG, ROPE),
                             QN > 1 ? 1 : kivi_waves(KB, VB, D, HG, ROPE) == 8 ? 2 : kivi_blocks_per_cu(KB, D, ROPE)) void kivi_mfma_kernel(MfmaParams p) {
  static_assert((KB == 2 || KB == 4) && (VB == 2 || VB == 4) && VB <= KB, "2- or 4-bit codes");
  static_assert(!ROPE || (KB == 2 && D <= 128), "rotary decode: 2-bit pages, head_dim <= 128");
  static_assert(2 * HG * QN <= 16, "hi and lo columns of the GQA group(s) fit one tile");
  static_assert(QN == 1 || (QN == 2 && HG == 4 && !ROPE), "two queries per block: GQA 4, keys without rotation");
  using PG = PageGeom<KB, VB, D>;
  constexpr int NW = kivi_waves(KB, VB, D, HG, ROPE);   // waves per block
  constexpr int NTH = 64 * NW;
  constexpr int KS = D / 32;             // k-steps of the key product
  constexpr int NT = D / 16;             // channel tiles of the value product
  constexpr int CPG = D / 4;             // key channels per lane group
  constexpr int KROW = D * KB / 8;       // bytes per key token row
  constexpr int CPR_K = KROW / 16;       // 16-byte chunks per key row
  constexpr int KW = CPG * KB / 32;      // key-code words per lane per 16-token tile
  constexpr int VROW = 32 * VB / 8;      // bytes per value channel column
  constexpr int GC = HG * QN;            // (query, head) pairs of the block
  constexpr int COMBOS = GC * 4 * KS;    // (pair, lane group, k-step) fold units
  constexpr int REPS = (COMBOS + 63) / 64;
  constexpr int PER_HEAD = 4 * KS;       // fold units (lanes) per head
  // bf16 B-operand sets for the residual keys (one per query when QN = 2)
  constexpr int QB = QN == 1 ? (3 * HG + 15) / 16 : QN;
  // the residual-key B operand is built once per wave and kept in registers
  // when it is small (QB * KS words of 16 bytes), else rebuilt for every step
  constexpr bool QPRE = !ROPE && QB * KS <= 4;
  static_assert(KW >= 1, "at least one word per lane");
  // B fragments of q' for the live columns (hi, lo): [column][(4 ks + g) ^ column]
  // in 16-byte slots; the XOR puts the 16 lanes that read one (ks, g) for
  // different columns, and the 16 lanes that write one column, on different
  // LDS banks (no padding)
  constexpr int FSTRIDE = 4 * KS;
  static_assert(FSTRIDE >= 8, "column slots cover the XOR range");
  constexpr int FRAG = 2 * GC * FSTRIDE * 16;
  // Per-wave LDS: [page buffer 0][page buffer 1][q' fragments]. A residual
  // step's 8 key + 8 value rows borrow page buffer 1 and the fragments: the
  // wave's first step is taken before its first page is computed (buffer 1 is
  // first filled for page 1, the fragments first written for page 0), any
  // further step after its last page.
  constexpr int WAVE_LDS = PG::NBUF * PG::BYTES + FRAG > PG::BYTES + PG::RING
                               ? PG::NBUF * PG::BYTES + FRAG : PG::BYTES + PG::RING;
  constexpr int RED = NW * GC * (D + 2) * 4;
  constexpr int ARENA = NW * WAVE_LDS > RED ? NW * WAVE_LDS : RED;

  __shared__ __attribute__((aligned(16))) float qs[GC][D];
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];              // per-wave areas / reduction
  // rotary decode: each wave's query rotated for the page in hand (row HG is
  // kept zero for the unused B columns), and omega_i / (2 pi) per channel pair
  __shared__ __attribute__((aligned(16))) float qpage[ROPE ? NW : 1][ROPE ? HG + 1 : 1][ROPE ? D : 4];
  __shared__ double w2pi[ROPE ? D / 2 : 1];
  __shared__ int last_block;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int j = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  // sequence b and its (first) query qi of the block
  const int rows_b = p.nq / QN;
  const int b = blockIdx.z / rows_b, qi = (blockIdx.z - b * rows_b) * QN;
  // lane column j of the key product: query j / (2HG), high part when
  // j % (2HG) < HG (then holding the scores of pair col_vh after the key
  // product); with one query only columns j < HG are live
  const bool col_hi = (j % (2 * HG)) < HG;
  const bool col_live = QN == 1 ? j < HG : col_hi;
  const int col_vh = (j / (2 * HG)) * HG + j % HG;
  const uint8_t* ringp = p.pm.ring(b, h);
  // tokens this sequence holds (a ragged batch: its own fill level, and its
  // own split between quantised pages and the ring)
  const int64_t fill = seq_len(p.seq_tokens, b, p.T);
  int64_t q_tokens = p.q_tokens;
  int32_t n_pages = p.n_pages, n_steps = p.n_steps;
  if (p.seq_tokens) {
    q_tokens = kivi_quantised(fill, p.residual);
    n_pages = static_cast<int32_t>(q_tokens / kPage);
  }
  // query qi of nq sits at position fill - nq + qi and sees the tokens up to
  // it: the pages and the ring up to its own token, or, when its token is in
  // a page, the pages up to that one (the rest of that page masked)
  // (with QN = 2 the block's second query sits one token later, at TbL - 1;
  // when every query's token is in a page the block takes the pages up to
  // the last one's and masks each column after its own query's token; when
  // the first query's token is the last quantised one, it sees every page
  // whole and only ring steps mask it)
  const int64_t Tb = fill - (p.nq - 1 - qi);
  const int64_t TbL = Tb + QN - 1;
  if (p.seq_tokens || p.nq > 1) n_steps = static_cast<int32_t>((TbL - q_tokens + 7) / 8);
  const bool in_page = TbL <= q_tokens;   // block-uniform: mask the rows' last pages
  if (in_page) {
    n_pages = static_cast<int32_t>((TbL + kPage - 1) / kPage);
    n_steps = 0;
  }
  uint8_t* wbuf = arena + wave * WAVE_LDS;
  uint32_t (*frag)[4] = reinterpret_cast<uint32_t (*)[4]>(wbuf + PG::NBUF * PG::BYTES);

  // (q staging and the first memory requests are issued below, after the
  // helpers they need are defined)

  // ---- per-wave online-softmax state ----------------------------------------
  // Lane (j, g), j < HG, tracks head j: running max m, and the sums of p and
  // p*z over its tokens (reduced over g at the end). acc rows 4g+r hold head
  // (4g+r) % HG: hi rows, then lo rows.
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_lane = -INFINITY, l_lane = 0.f, z_lane = 0.f;

  // Folds NS scores per lane into the softmax state (rescaling the running
  // sums and accumulators if a head's max grows); turns s into weights 2^(s-m).
  auto softmax_update = [&](float* s, auto ns_tag) {
    constexpr int NS = decltype(ns_tag)::value;
    float pmax = s[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) pmax = fmaxf(pmax, s[i]);
    // the reference max moves only when a score exceeds it by more than
    // kMaxSlack (weights stay below 2^kMaxSlack; any reference gives the same
    // softmax), so the accumulators are rarely rescaled. A head's scores are
    // spread over its four lane groups; whether any of them exceeds the slack
    // is decided by each lane's own maximum, so the maximum over the lane
    // groups is only formed on the rare rescaling pages.
    const bool grows = col_live && (pmax > m_lane + kMaxSlack);
    if (__builtin_amdgcn_ballot_w64(grows) != 0) {   // wave-uniform
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      const float m_new = fmaxf(m_lane, pmax);
      // a column whose max stays keeps its sums (also one that has seen no
      // token yet, -inf: with two queries per block the other query's
      // columns may move while this one stays there)
      const float alpha = m_new == m_lane ? 1.0f : fast_exp2(m_lane - m_new);
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
    for (int i = 0; i < NS; ++i) s[i] = fast_exp2(s[i] - m_lane);
  };

  // ---- work of this wave --------------------------------------------------------
  // Block `split` takes a contiguous range of pages; its waves take every
  // NW-th page of that range.
  const int waves_total = p.splits * NW;
  const int pg0 = static_cast<int>(static_cast<int64_t>(split) * n_pages / p.splits);
  const int pg1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_pages / p.splits);
  const int n_mine = pg0 + wave < pg1 ? (pg1 - pg0 - wave + NW - 1) / NW : 0;

  float qreg[REPS][8];   // this lane's fold units of q (set once q is staged)
  // rotary decode: this lane's channel pairs are (D/8) g + m, m < D/8; rcos/rsin
  // hold the rotation of tile row j (token 16 mt + j of a page) by omega_i, and
  // qpair this lane's pair (lane) of every head's query
  constexpr int NPL = ROPE ? D / 8 : 1;
  float rcos[2][NPL], rsin[2][NPL], qpair[HG][2];

  // qpage[wave][hh] = R(omega (T-1-t0)) q[hh]: scores of keys at t0 + j are then
  // qpage . R(omega j) k (the rotations of query and key combine into one by
  // the relative position)
  auto rotate_q = [&](int64_t t0) {
    if (lane < D / 2) {
      const double turns = static_cast<double>(Tb - 1 - t0) * w2pi[lane];
      float sn, cs;
      sincospif(2.0f * static_cast<float>(turns - floor(turns)), &sn, &cs);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float q0 = qpair[hh][0], q1 = qpair[hh][1];
        *reinterpret_cast<float2*>(&qpage[wave][hh][2 * lane]) = float2{q0 * cs - q1 * sn, q0 * sn + q1 * cs};
      }
    }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  };
  // B values of the fp32 key product for this lane: column j is head j (or zero)
  auto load_bq = [&](float* bqv) {
    const float* src = &qpage[wave][j < HG ? j : HG][(D / 4) * g];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(src + 4 * i);
      bqv[4 * i] = v.x;
      bqv[4 * i + 1] = v.y;
      bqv[4 * i + 2] = v.z;
      bqv[4 * i + 3] = v.w;
    }
  };
  // y (this lane's D/4 channels, dequantised) -> R(omega tau) y, pair by pair
  auto rotate_keys = [&](float* y, int mt) {
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      const float x0 = y[2 * m], x1 = y[2 * m + 1];
      const float c = rcos[mt][m], sn = rsin[mt][m];
      y[2 * m] = x0 * c - x1 * sn;
      y[2 * m + 1] = x0 * sn + x1 * c;
    }
  };

  auto issue_page = [&](int k) {   // page k of this wave -> buffer k % NBUF
    const uint8_t* src = p.pm.page(b, h, pg0 + wave + NW * k);
    const uint32_t dst = lds_addr(wbuf + (k % PG::NBUF) * PG::BYTES);
#pragma unroll
    for (int i = 0; i < PG::DMA; ++i) {
      const int off = i * 1024 + lane * 16;
      int from = off;   // key rows: chunk permutation (see kswz)
      if (off < PG::CODES) from = krow_off<CPR_K>(off / KROW, off % KROW);
      if (i + 1 < PG::DMA || off < PG::BYTES) dma16(src + from, dst + i * 1024);
    }
  };

  auto process_page = [&](const uint8_t* pg, int64_t t0) {
    float s[8];
    if constexpr (ROPE) {
      // scores of tile row j = qpage . R(omega tau) (code * s + z), tau = 16 mt + j,
      // on v_mfma_f32_16x16x4f32 (lane group g holds channels (D/4) g ..)
      rotate_q(t0);
      float bqv[D / 4], sv[D / 4], zv[D / 4];
      load_bq(bqv);
      const float* sp = reinterpret_cast<const float*>(pg + PG::OFF_KS) + (D / 4) * g;
      const float* zp = reinterpret_cast<const float*>(pg + PG::OFF_KZ) + (D / 4) * g;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(sp + 4 * i);
        const float4 c = *reinterpret_cast<const float4*>(zp + 4 * i);
        sv[4 * i] = a.x; sv[4 * i + 1] = a.y; sv[4 * i + 2] = a.z; sv[4 * i + 3] = a.w;
        zv[4 * i] = c.x; zv[4 * i + 1] = c.y; zv[4 * i + 2] = c.z; zv[4 * i + 3] = c.w;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float y[D / 4];
#pragma unroll
        for (int w = 0; w < D / 64; ++w) {
          const uint32_t word =
              *reinterpret_cast<const uint32_t*>(pg + krow_off<CPR_K>(tile_tok<ROPE>(mt, j), (D / 16) * g + 4 * w));
#pragma unroll
          for (int c = 0; c < 16; ++c)
            y[16 * w + c] = fmaf(static_cast<float>((word >> (2 * c)) & 3u), sv[16 * w + c], zv[16 * w + c]);
        }
        rotate_keys(y, mt);
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 4; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x4f32(y[ks], bqv[ks], c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * mt + r] = c[r];
      }
    } else {
    // q' = q * s per channel, split hi/lo into B fragments; bias q . z
    float bias_part[REPS];
    float amax = 0.f;   // largest |q'| of the lane (f16 range check below)
    // (scaled by 2^-esc: 0 except on the rare pages described below)
    auto fold = [&](int r, int esc_, bool with_bias) {
      const int cidx = lane + 64 * r;
      const int fh = cidx / PER_HEAD, fg = (cidx / KS) % 4, fk = cidx % KS;
      const int c0 = fg * CPG + 8 * fk;
      const int chi = (fh / HG) * 2 * HG + fh % HG, clo = chi + HG;   // B columns of pair fh
      const float4 s0 = *reinterpret_cast<const float4*>(pg + PG::OFF_KS + 4 * c0);
      const float4 s1 = *reinterpret_cast<const float4*>(pg + PG::OFF_KS + 4 * c0 + 16);
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float qp[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qp[i] = qreg[r][i] * sv[i];
        amax = fmaxf(amax, fabsf(qp[i]));
        if (esc_) qp[i] = ldexpf(qp[i], -esc_);
      }
      if (with_bias) {
        const float4 z0 = *reinterpret_cast<const float4*>(pg + PG::OFF_KZ + 4 * c0);
        const float4 z1 = *reinterpret_cast<const float4*>(pg + PG::OFF_KZ + 4 * c0 + 16);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        float bp = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) bp = fmaf(qreg[r][i], zv[i], bp);
        bias_part[r] = bp;
      }
      uint32_t hi[4], lo[4];   // fragment order {0,2,1,3,4,6,5,7}
      split_f16(qp[0], qp[2], hi[0], lo[0]);
      split_f16(qp[1], qp[3], hi[1], lo[1]);
      split_f16(qp[4], qp[6], hi[2], lo[2]);
      split_f16(qp[5], qp[7], hi[3], lo[3]);
      if (cidx < COMBOS) {
        *reinterpret_cast<uint4*>(frag[chi * FSTRIDE + ((4 * fk + fg) ^ (chi & 7))]) =
            uint4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<uint4*>(frag[clo * FSTRIDE + ((4 * fk + fg) ^ (clo & 7))]) =
            uint4{lo[0], lo[1], lo[2], lo[3]};
      }
    };
#pragma unroll
    for (int r = 0; r < REPS; ++r) fold(r, 0, true);
    // f16 range of the key operand: beyond 65504 the f16 high part saturates.
    // A page whose q' exceeds it (a key channel with an enormous range) folds
    // again with q' 2^-e (e from the wave's largest |q'|), overwriting the
    // fragments, and multiplies the product part of its scores by 2^e:
    // exact scaling by a power of two (wave-uniform, rare).
    const bool big = __builtin_amdgcn_ballot_w64(amax > 65504.f) != 0;
    int esc = 0;
    if (big) {
      const float wm = wave_max(amax);
      int ex;
      frexpf(wm, &ex);   // wm < 2^ex
      esc = __builtin_amdgcn_readfirstlane(ex - 15);
#pragma unroll
      for (int r = 0; r < REPS; ++r) fold(r, esc, false);
    }
    // bias of head j for this lane: the fold units of head hh are lanes
    // [PER_HEAD*hh, PER_HEAD*(hh+1)) counted across reps of 64
    float bias_j = 0.f;
#pragma unroll
    for (int r = 0; r < REPS; ++r) {
      float v = bias_part[r];
      if constexpr (PER_HEAD == 8) {
        v = sum8(v);
      } else {
        v = row_sum16(v);
        if constexpr (PER_HEAD == 32) v += xor16(v);
      }
      const int src = PER_HEAD * (col_live ? col_vh : 0) - 64 * r;
      const float got = __shfl(v, src & 63, 64);
      if (src >= 0 && src < 64) bias_j = got;
    }
    if (!col_live) bias_j = 0.f;   // lo columns carry no offset
    if (big) bias_j = ldexpf(bias_j, -esc);   // scaled with the product, undone below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // (with one query, columns >= 2*HG only produce score columns that are
    // never read)
    half8 bq[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int col = j % (2 * GC);
      const uint4 f = *reinterpret_cast<const uint4*>(frag[col * FSTRIDE + ((4 * ks + g) ^ (col & 7))]);
      bq[ks] = cat4h(f.x, f.y, f.z, f.w);
    }

    // scores S^T = codes x q'^T
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      uint32_t kp[KW];
#pragma unroll
      for (int w = 0; w < KW; ++w)
        kp[w] = *reinterpret_cast<const uint32_t*>(pg + krow_off<CPR_K>(tile_tok<ROPE>(mt, j), g * (KW * 4) + 4 * w));
      floatx4 c = {bias_j, bias_j, bias_j, bias_j};   // hi column carries q . z
      if constexpr (KB == 2) {
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          half8 a0, a1;
          codes2_frags(kp[w], a0, a1);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bq[2 * w], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bq[2 * w + 1], c, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int w = 0; w < KW; ++w)
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes4_frag(kp[w]), bq[w], c, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * mt + r] = c[r] + row_shl<HG>(c[r]);
    }
    if (big) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = ldexpf(s[i], esc);
    }
    }   // rotary / plain keys

    // a query's own token is in this page (or, with two queries, the first
    // query's last token is on the page before): each column masks the tokens
    // after its own query's (wave-uniform check)
    const bool masked_page = in_page && Tb - t0 < kPage;
    const int nvalid = static_cast<int>(Tb + (QN == 1 ? 0 : j / (2 * HG)) - t0);
    if (masked_page) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile_tok<ROPE>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = -INFINITY;
    }
    softmax_update(s, std::integral_constant<int, 8>{});
    if constexpr (QN == 2) {
      // the first query may have no token in the page, and a wave that has
      // seen none of its tokens yet has reference max -inf: weight 0
      if (masked_page) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (tile_tok<ROPE>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = 0.f;
      }
    }
    // per-token value scale and offset of this lane's tokens tile_tok(mt, 4g + r)
    constexpr int VT0 = ROPE ? 16 : 32, VT1 = ROPE ? 64 : 16;
    const float4 vs0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + VT0 * g);
    const float4 vs1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + VT1 + VT0 * g);
    const float4 vz0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + VT0 * g);
    const float4 vz1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + VT1 + VT0 * g);
    const float vsv[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    const float vzv[8] = {vz0.x, vz0.y, vz0.z, vz0.w, vz1.x, vz1.y, vz1.z, vz1.w};
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      l_lane += s[i];
      z_lane = fmaf(s[i], vzv[i], z_lane);
      pv[i] = s[i] * vsv[i];
    }
    // P' into A fragments: the lane's tokens in the order {0,2,1,3,4,6,5,7}
    uint32_t ph[4], pl[4];
    split_bf16(pv[0], pv[2], ph[0], pl[0]);
    split_bf16(pv[1], pv[3], ph[1], pl[1]);
    split_bf16(pv[4], pv[6], ph[2], pl[2]);
    split_bf16(pv[5], pv[7], ph[3], pl[3]);
    // rows j < HG: hi of head j; rows j >= HG: lo of lane j-HG (rows >= 2HG
    // only reach accumulator rows that are never read)
    // (QN = 2: the second query's high rows 2HG.. keep their own values)
    uint32_t pa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = shr_keep<HG>(ph[i], pl[i]);
      if constexpr (QN == 2) pa[i] = col_hi ? ph[i] : pa[i];
    }
    const bf16x8 ap = __builtin_bit_cast(bf16x8, uint4{pa[0], pa[1], pa[2], pa[3]});

    // P' x value codes; channel of N-tile nt in column j is 16 nt + j (adjacent
    // lanes read adjacent value columns: no LDS bank conflicts). Lane group g
    // needs tokens 8g..8g+7 of a column: 16 bits of a 2-bit column, 32 of a
    // 4-bit one; the converts give them in the order {0,2,1,3,4,6,5,7} of P'.
    if constexpr (ROPE) {   // 2-bit values, tokens 4g..4g+3 and 16+4g..16+4g+3
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint2 v2 = *reinterpret_cast<const uint2*>(pg + PG::OFF_VC + (16 * nt + j) * VROW);
        // byte g of each word
        const uint32_t x = __builtin_amdgcn_perm(v2.y, v2.x, 0x0C0C0400u + 0x0101u * g);
        const uint32_t y0 = x & 0x3333u, y1 = (x >> 2) & 0x3333u;
        const uint4 bw{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 0)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 0)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 1)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 1))};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
      }
    } else if constexpr (VB == 2) {
#pragma unroll
      for (int nt = 0; nt < NT; nt += 2) {   // two channel tiles per code word
        const uint8_t* col = pg + PG::OFF_VC + (16 * nt + j) * VROW + 2 * g;
        u16x2 xv;
        xv.x = *reinterpret_cast<const uint16_t*>(col);
        xv.y = *reinterpret_cast<const uint16_t*>(col + 16 * VROW);
        const uint32_t x = __builtin_bit_cast(uint32_t, xv);
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
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(pg + PG::OFF_VC + (16 * nt + j) * VROW + 4 * g);
        const uint32_t y0 = w & 0x0F0F0F0Fu, y1 = (w >> 4) & 0x0F0F0F0Fu;
        const uint4 bw{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, false)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, false)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, true)),
                       bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, true))};
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
      }
    }
  };

  // ---- residual (unquantised) tokens, 8 per step ----------------------------
  // Step hs covers tokens [q_tokens + 8 hs, +8); the steps of this (sequence,
  // KV head) are spread over all its waves. Rows go HBM -> LDS slot `wring`.
  uint8_t* wring = wbuf + PG::BYTES;
  constexpr int LPR = 2 * D / 16;           // lanes per bf16 row
  constexpr int RPI = 64 / LPR;             // rows per 16-byte-per-lane copy
  constexpr int RSTEP = 8;                  // tokens per residual step
  bool owns_new = false;   // this wave's step holds the token appended by this call
  // the appended token's K and V rows as byte offsets from the ring (plain
  // integers: a per-lane choice between two pointers read from the
  // parameters would be compiled into an indexed stack load)
  const int64_t new_row = (static_cast<int64_t>(b) * p.kv_heads + h) * (2 * D);
  const int64_t new_off[2] = {
      static_cast<int64_t>(reinterpret_cast<uintptr_t>(p.k_new) - reinterpret_cast<uintptr_t>(ringp)) + new_row,
      static_cast<int64_t>(reinterpret_cast<uintptr_t>(p.v_new) - reinterpret_cast<uintptr_t>(ringp)) + new_row};
  auto issue_step = [&](int hs) -> int {    // returns the copies issued
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    const int nv = static_cast<int>(TbL - t0 < RSTEP ? TbL - t0 : RSTEP);   // rows up to the last query's token
    const int row_in = lane / LPR, col_b = (lane % LPR) * 16;
    const int slots = static_cast<int>(p.ring_slots);
    const int slot0 = static_cast<int>(t0 % p.ring_slots);
    // the appended token's row comes from the input (its ring slot is written below)
    const int64_t rnew = p.new_tok - t0;
    if (rnew >= 0 && rnew < RSTEP) owns_new = true;
    int issued = 0;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
      for (int i = 0; i < (RSTEP + RPI - 1) / RPI; ++i) {
        if (i * RPI >= nv) continue;          // wave-uniform: no row of this copy exists
        const int r = i * RPI + row_in;
        const int slot = slot0 + r < slots ? slot0 + r : slot0 + r - slots;
        const int64_t off = r == rnew ? new_off[kv] : (kv * p.ring_slots + slot) * (2 * D);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(ringp) + off + col_b);
        if (r < nv && r < RSTEP) dma16(src, lds_addr(wring + kv * RSTEP * 2 * D + i * 1024));
        ++issued;
      }
    }
    // value rows of absent tokens must be finite (they meet weight 0): zero them
    for (int i = lane; i < (RSTEP - nv) * 2 * D / 16; i += 64)
      *reinterpret_cast<uint4*>(wring + RSTEP * 2 * D + nv * 2 * D + i * 16) = uint4{0u, 0u, 0u, 0u};
    return issued;
  };
  uint4 qstep[QPRE ? QB : 1][QPRE ? KS : 1];
  // B operand of the residual key product: q^T in three bf16 parts, columns
  // [0,HG) hi, [HG,2HG) mid, [2HG,3HG) lo, the rest zero (from the scaled q in qs)
  // (QN = 2: set qb is query qb's, the same 3HG columns)
  auto qstep_operand = [&](int qb, int ks) -> uint4 {
    const int col = QN == 1 ? 16 * qb + j : j;
    const int part = col / HG, hh = (QN == 1 ? 0 : qb * HG) + col % HG;
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 qq = *reinterpret_cast<const float2*>(&qs[hh][32 * ks + 8 * g + 2 * i]);
      const float h0 = bf16_trunc(qq.x), h1 = bf16_trunc(qq.y);
      const float m0 = bf16_trunc(qq.x - h0), m1 = bf16_trunc(qq.y - h1);
      float x0 = part == 0 ? h0 : (part == 1 ? m0 : qq.x - h0 - m0);
      float x1 = part == 0 ? h1 : (part == 1 ? m1 : qq.y - h1 - m1);
      if (part >= 3) x0 = x1 = 0.f;      // unused columns
      w4[i] = pack_bf16(x0, x1);
    }
    return uint4{w4[0], w4[1], w4[2], w4[3]};
  };
  // tile rows (tokens) 8..15 of a step are masked; key rows repeat rows 0..7
  auto process_step = [&](int hs) {
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    // tokens of the step this lane's column sees (its query's own count)
    const int64_t Tj = Tb + (QN == 1 ? 0 : j / (2 * HG));
    const int nv = static_cast<int>(Tj - t0 < RSTEP ? Tj - t0 : RSTEP);
    float sc[4];
    if constexpr (ROPE) {
      // key rows rotated by their position in the step, fp32 product as for pages
      rotate_q(t0);
      float bqv[D / 4], y[D / 4];
      load_bq(bqv);
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(wring + (j & 7) * 2 * D) + (D / 4) * g;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + 8 * i);
        unpack_bf16x8(v, y + 8 * i);
      }
      rotate_keys(y, 0);
      floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 4; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x4f32(y[ks], bqv[ks], c, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (4 * g + r < nv) ? c[r] : -INFINITY;
    } else {
    floatx4 cres[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) cres[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wring + (j & 7) * 2 * D + (32 * ks + 8 * g) * 2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        uint4 w;
        if constexpr (QPRE) w = qstep[QPRE ? qb : 0][QPRE ? ks : 0];
        else w = qstep_operand(qb, ks);
        cres[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, w), cres[qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v;
      if constexpr (QN == 2) {   // query q's sums in lanes < HG of set q; set 1 moves to columns 2HG..
        const float v0 = cres[0][r] + row_shl<HG>(cres[0][r]) + row_shl<2 * HG>(cres[0][r]);
        const float v1 = cres[1][r] + row_shl<HG>(cres[1][r]) + row_shl<2 * HG>(cres[1][r]);
        v = __uint_as_float(shr_keep<2 * HG>(__float_as_uint(v0), __float_as_uint(v1)));
      } else if constexpr (3 * HG <= 16) {
        v = cres[0][r] + row_shl<HG>(cres[0][r]) + row_shl<2 * HG>(cres[0][r]);
      } else {   // HG = 8: hi and mid in set 0, lo in set 1
        v = cres[0][r] + row_shl<HG>(cres[0][r]) + cres[QB - 1][r];
      }
      sc[r] = (4 * g + r < nv) ? v : -INFINITY;
    }
    }   // rotary / plain keys
    softmax_update(sc, std::integral_constant<int, 4>{});
    if constexpr (QN == 2) {
      // the block's steps reach its second query's token, so a step may hold
      // none of the first query's tokens; in a wave that has seen no token of
      // it yet (reference max still -inf) 2^(-inf - -inf) is not 0: absent
      // tokens get weight 0 explicitly
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = 4 * g + r < nv ? sc[r] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) l_lane += sc[r];   // absent tokens contribute 0
    // P in bf16 hi/lo rows; k index 8g+i holds token 4g+i for i < 4, zero after
    uint32_t ph[2], pl[2];
    split_bf16(sc[0], sc[1], ph[0], pl[0]);
    split_bf16(sc[2], sc[3], ph[1], pl[1]);
    uint32_t pa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      pa[i] = shr_keep<HG>(ph[i], pl[i]);
      if constexpr (QN == 2) pa[i] = col_hi ? ph[i] : pa[i];
    }
    const bf16x8 ap = __builtin_bit_cast(bf16x8, uint4{pa[0], pa[1], 0u, 0u});
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = 16 * nt + j;
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(wring + RSTEP * 2 * D) + c;
      const int t4 = (4 * g) & 7;             // tokens >= 8 carry weight 0
      const uint32_t v0 = vr[(t4 + 0) * D], v1 = vr[(t4 + 1) * D];
      const uint32_t v2 = vr[(t4 + 2) * D], v3 = vr[(t4 + 3) * D];
      const bf16x8 bv = __builtin_bit_cast(bf16x8, uint4{v0 | (v1 << 16), v2 | (v3 << 16), 0u, 0u});
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bv, acc[nt], 0, 0, 0);
    }
  };

  // ---- first requests, all in flight together: q (wave 0), this wave's first
  // residual step, its first page ------------------------------------------------
  // residual steps go first to the waves with the fewest pages: the last wave
  // of every block, then the one before, ... (wave 0 may hold one page more)
  const int my_wave = (NW - 1 - wave) * p.splits + split;
  const int q_bytes = HG * D * (p.q_bf16 ? 2 : 4);   // one query's heads of this KV head
  int after_q = 0;
  if (wave == 0) {
#pragma unroll
    for (int qq = 0; qq < QN; ++qq) {   // raw rows of the block's queries, one after the other
      const uint8_t* qsrc = p.q + (static_cast<int64_t>(b * p.nq + qi + qq) * p.q_heads + h * HG) * D * (p.q_bf16 ? 2 : 4);
      for (int off = 0; off < q_bytes; off += 1024)
        if (off + lane * 16 < q_bytes) dma16(qsrc + off + lane * 16, lds_addr(&qs[0][0]) + qq * q_bytes + off);
    }
  }
  const bool has_step = my_wave < n_steps;
  if (has_step) after_q += issue_step(my_wave);
  if (n_mine > 0) {
    issue_page(0);
    after_q += PG::DMA;
  }
  if constexpr (ROPE) {
    for (int i = tid; i < D / 2; i += NTH)
      w2pi[i] = pow(p.rope_theta, -2.0 * i / D) * 0.15915494309189535;   // omega_i / (2 pi)
    for (int i = lane; i < D; i += 64) qpage[wave][HG][i] = 0.f;
  }
  if (wave == 0) wait_vm_upto(after_q);   // q has landed
  __syncthreads();
  {
    // raw query (bf16 or f32) -> f32 * sm_scale * log2(e), in place
    constexpr int PER = (GC * D + NTH - 1) / NTH;
    float qv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      qv[k] = 0.f;
      if (i < GC * D)
        qv[k] = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(&qs[0][0])[i])
                         : (&qs[0][0])[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      if (i < GC * D) (&qs[0][0])[i] = qv[k] * p.qscale;
    }
    __syncthreads();
  }
  if constexpr (ROPE) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int m = 0; m < NPL; ++m) {
        const double turns = static_cast<double>(tile_tok<ROPE>(mt, j)) * w2pi[(D / 8) * g + m];
        sincospif(2.0f * static_cast<float>(turns - floor(turns)), &rsin[mt][m], &rcos[mt][m]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      qpair[hh][0] = lane < D / 2 ? qs[hh][2 * lane] : 0.f;
      qpair[hh][1] = lane < D / 2 ? qs[hh][2 * lane + 1] : 0.f;
    }
  }
  if constexpr (QPRE) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qstep[qb][ks] = qstep_operand(qb, ks);
  }
  // fold units handled by this lane: (head, lane group, k-step) -> 8 channels
#pragma unroll
  for (int r = 0; r < REPS; ++r) {
    const int cidx = lane + 64 * r;
    const int fh = cidx / PER_HEAD, fg = (cidx / KS) % 4, fk = cidx % KS;
    const int c0 = fg * CPG + 8 * fk;
#pragma unroll
    for (int i = 0; i < 8; ++i) qreg[r][i] = cidx < COMBOS ? qs[fh][c0 + i] : 0.f;
  }
  if (has_step) {
    if (n_mine > 0) wait_vm<PG::DMA>();   // the first page may stay in flight
    else wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    process_step(my_wave);
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  }

  // ---- pages: DMA pipeline, one page ahead (page 0 already requested) --------
#pragma unroll 1
  for (int k = 0; k < n_mine; ++k) {
    // waves with more pages left issue first: the waves of a SIMD (from
    // different blocks) then finish their pages together instead of the
    // oldest first, leaving the last one alone on the SIMD
    {
      const int rem = n_mine - k;
      if (rem >= 4) __builtin_amdgcn_s_setprio(2);
      else if (rem >= 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    wait_lds();   // the buffer about to be refilled has been read
    __builtin_amdgcn_wave_barrier();
    const bool next = k + 1 < n_mine;
    if (next) issue_page(k + 1);
    if (next) wait_vm<PG::DMA>();
    else wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    process_page(wbuf + (k % PG::NBUF) * PG::BYTES,
                 static_cast<int64_t>(pg0 + wave + NW * k) * kPage);
  }

  // ---- any further residual steps of this wave (when steps outnumber waves) --
#pragma unroll 1
  for (int hs = my_wave + waves_total; hs < n_steps; hs += waves_total) {
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    issue_step(hs);
    wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    process_step(hs);
  }
  wait_lds();
  // the appended token's K and V rows into its ring slot (one wave per
  // (sequence, KV head) takes its step); the merge's wait or the kernel's end
  // completes the stores
  if (owns_new && lane < 2 * (2 * D / 16)) {
    const int kv = lane / (2 * D / 16), c16 = lane % (2 * D / 16);
    const int64_t slot = p.new_tok % p.ring_slots;
    const uint8_t* src = (kv ? p.v_new : p.k_new) + (static_cast<int64_t>(b) * p.kv_heads + h) * (2 * D) + 16 * c16;
    uint8_t* dst = const_cast<uint8_t*>(ringp) + (kv * p.ring_slots + slot) * (2 * D) + 16 * c16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  __builtin_amdgcn_s_setprio(3);   // the epilogue and merge end the block's critical path
  // ---- wave epilogue -----------------------------------------------------------
  // per (query, head) pair vh: its column (vh / HG) 2HG + vh % HG
  float lsum[GC], zsum[GC], mh[GC];
  {
    float l_ = l_lane, z_ = z_lane;
    l_ += xor16(l_);
    l_ += xor32(l_);
    z_ += xor16(z_);
    z_ += xor32(z_);
#pragma unroll
    for (int vh = 0; vh < GC; ++vh) {
      const int col = (vh / HG) * 2 * HG + vh % HG;
      lsum[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_), col));
      zsum[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z_), col));
      mh[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_lane), col));
    }
  }
  finish_unit<D, HG, NW, QN>(p, acc, mh, lsum, zsum, arena, last_block, b, qi, h, split);
}

// ---- four queries per block over dequantised keys (GQA 4) -----------------------
// Four consecutive queries of a sequence per block: their 16 (query, head)
// pairs are the 16 columns of the key product and the 16 rows of the value
// product. Each page's keys are dequantised in registers (code * s + z per
// channel, in fp32) straight into the f16 high and remainder parts of the A
// operand, and the query's parts (high and remainder of q', built once) are
// the B operand: three products per k-step, Kh Qh + Kl Qh + Kh Ql. The page
// work that grows with the queries is then the softmax and the weights only;
// kivi_mfma_kernel instead folds the page's key scales into every query's
// columns, work that grows with each query. f16 range: q' and the page's
// keys are scaled by powers of two below 2^15 (exact; the page's bound is
// max(|z|, |z + (2^KB - 1) s|) over its channels), undone on the scores.
// Residual tokens: the bf16 key rows against q' in three bf16 parts, as in
// kivi_mfma_kernel. Uniform batches only (one fill level).
template <int KB, int VB, int D>
__global__ __launch_bounds__(512, 1) void kivi_deq_kernel(MfmaParams p) {
  static_assert((KB == 2 || KB == 4) && (VB == 2 || VB == 4) && VB <= KB && D <= 128,
                "2- or 4-bit keys, 2- or 4-bit values, d <= 128");
  constexpr int HG = 4, QN = 4, GC = HG * QN;   // 16 (query, head) pairs
  constexpr int NW = 8, NTH = 64 * NW;
  using PG = PageGeom<KB, VB, D>;
  constexpr int KS = D / 32;             // k-steps of the key product
  constexpr int NT = D / 16;             // channel tiles of the value product
  constexpr int CPG = D / 4;             // key channels per lane group
  constexpr int KROW = D * KB / 8;       // bytes per key token row
  constexpr int CPR_K = KROW / 16;
  constexpr int FPW = 32 / KB;           // codes per 32-bit word
  constexpr int KW = CPG / FPW;          // key-code words per lane per 16-token tile
  constexpr int VROW = 32 * VB / 8;
  constexpr float kLevels = float((1 << KB) - 1);
  // per-wave LDS: two page buffers; a residual step's 8 key + 8 value rows
  // borrow page buffer 1 (and what follows) before the first page and after
  // the last
  constexpr int WAVE_LDS = 2 * PG::BYTES > PG::BYTES + PG::RING ? 2 * PG::BYTES : PG::BYTES + PG::RING;
  constexpr int RED = NW * GC * (D + 2) * 4;
  constexpr int ARENA = NW * WAVE_LDS > RED ? NW * WAVE_LDS : RED;
  __shared__ __attribute__((aligned(16))) float qs[GC][D];
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];
  __shared__ int last_block;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y;
  const int rows_b = p.nq / QN;
  const int b = blockIdx.z / rows_b, qi = (blockIdx.z - b * rows_b) * QN;
  const uint8_t* ringp = p.pm.ring(b, h);
  // column j: query j / HG of the block (at position Tb - 1 + j / HG), head j % HG
  const int64_t q_tokens = p.q_tokens;
  const int64_t Tb = p.T - (p.nq - 1 - qi);   // tokens the block's first query sees
  const int64_t TbL = Tb + QN - 1;            // ... and its last
  int32_t n_pages = p.n_pages;
  int32_t n_steps = static_cast<int32_t>((TbL - q_tokens + 7) / 8);
  const bool in_page = TbL <= q_tokens;
  if (in_page) {
    n_pages = static_cast<int32_t>((TbL + kPage - 1) / kPage);
    n_steps = 0;
  }
  const int64_t Tj = Tb + j / HG;             // tokens column j's query sees
  uint8_t* wbuf = arena + wave * WAVE_LDS;

  floatx4 acc[NT];   // rows 4g + r: pair 4g + r
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_lane = -INFINITY, l_lane = 0.f, z_lane = 0.f;   // column j (summed over g at the end)

  auto softmax_update = [&](float* s, auto ns_tag) {
    constexpr int NS = decltype(ns_tag)::value;
    float pmax = s[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) pmax = fmaxf(pmax, s[i]);
    const bool grows = pmax > m_lane + kMaxSlack;
    if (__builtin_amdgcn_ballot_w64(grows) != 0) {   // wave-uniform
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      const float m_new = fmaxf(m_lane, pmax);
      const float alpha = m_new == m_lane ? 1.0f : fast_exp2(m_lane - m_new);
      l_lane *= alpha;
      z_lane *= alpha;
      m_lane = m_new;
      // accumulator row 4g + r is pair 4g + r: its factor from lane 4g + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= a;
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) s[i] = fast_exp2(s[i] - m_lane);
  };

  // ---- this wave's pages: block `split` takes a contiguous range, its waves
  // every NW-th page of it ---------------------------------------------------
  const int waves_total = p.splits * NW;
  const int pg0 = static_cast<int>(static_cast<int64_t>(split) * n_pages / p.splits);
  const int pg1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_pages / p.splits);
  const int n_mine = pg0 + wave < pg1 ? (pg1 - pg0 - wave + NW - 1) / NW : 0;

  auto issue_page = [&](int k) {   // page k of this wave -> buffer k % 2
    const uint8_t* src = p.pm.page(b, h, pg0 + wave + NW * k);
    const uint32_t dst = lds_addr(wbuf + (k % 2) * PG::BYTES);
#pragma unroll
    for (int i = 0; i < PG::DMA; ++i) {
      const int off = i * 1024 + lane * 16;
      int from = off;
      if (off < PG::CODES) from = krow_off<CPR_K>(off / KROW, off % KROW);
      if (i + 1 < PG::DMA || off < PG::BYTES) dma16(src + from, dst + i * 1024);
    }
  };

  // B operand of the key product (q' of pair j, scaled by 2^-eq), for k-step
  // ks and lane group g: channels g CPG + 8 ks + {0,2,1,3,4,6,5,7}, the order
  // in which the key fragments below are built
  half8 bqh[KS], bql[KS];
  int eq = 0;

  // one word of key codes -> its FPW codes as f32, field order
  auto codes_f32 = [&](uint32_t wd, float* x) {
    if constexpr (KB == 2) {
      const uint32_t y0 = wd & 0x33333333u, y1 = (wd >> 2) & 0x33333333u;
      // byte SEL of y0 holds fields 4 SEL, 4 SEL + 2; of y1 fields 4 SEL + 1, 4 SEL + 3
      const float2 a0 = codes2_f32<0>(y0), a1 = codes2_f32<0>(y1);
      const float2 a2 = codes2_f32<1>(y0), a3 = codes2_f32<1>(y1);
      const float2 a4 = codes2_f32<2>(y0), a5 = codes2_f32<2>(y1);
      const float2 a6 = codes2_f32<3>(y0), a7 = codes2_f32<3>(y1);
      x[0] = a0.x; x[2] = a0.y; x[1] = a1.x; x[3] = a1.y;
      x[4] = a2.x; x[6] = a2.y; x[5] = a3.x; x[7] = a3.y;
      x[8] = a4.x; x[10] = a4.y; x[9] = a5.x; x[11] = a5.y;
      x[12] = a6.x; x[14] = a6.y; x[13] = a7.x; x[15] = a7.y;
    } else {
      // nibbles -> bytes: byte k of y0 holds field 2k, of y1 field 2k + 1
      const uint32_t y0 = wd & 0x0F0F0F0Fu, y1 = (wd >> 4) & 0x0F0F0F0Fu;
      const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y0, 512.0f, false);
      const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y1, 512.0f, false);
      const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y0, 512.0f, true);
      const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y1, 512.0f, true);
      x[0] = a0[0]; x[2] = a0[1]; x[1] = a1[0]; x[3] = a1[1];
      x[4] = a2[0]; x[6] = a2[1]; x[5] = a3[0]; x[7] = a3[1];
    }
  };

  auto process_page = [&](const uint8_t* pg, int64_t t0) {
    // f16 range of the page's keys: |code s + z| <= max(|z|, |z + levels s|)
    float kb = 0.f;
#pragma unroll
    for (int c = lane; c < D; c += 64) {
      const float sc = reinterpret_cast<const float*>(pg + PG::OFF_KS)[c];
      const float zc = reinterpret_cast<const float*>(pg + PG::OFF_KZ)[c];
      kb = fmaxf(kb, fmaxf(fabsf(zc), fabsf(fmaf(kLevels, sc, zc))));
    }
    int ek = 0;
    if (__builtin_amdgcn_ballot_w64(kb >= 32768.f) != 0) {   // rare: keys beyond 2^15
      int ex;
      frexpf(wave_max(kb), &ex);
      ek = __builtin_amdgcn_readfirstlane(ex - 15);
    }
    uint32_t kp[2][KW];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int w = 0; w < KW; ++w)
        kp[mt][w] = *reinterpret_cast<const uint32_t*>(pg + krow_off<CPR_K>(tile_tok<false>(mt, j), g * (KW * 4) + 4 * w));
    floatx4 c[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int w = 0; w < KW; ++w) {
      // scale and offset of this word's FPW channels g CPG + FPW w + i
      const int cw = g * CPG + FPW * w;
      float sv[FPW], zv[FPW];
#pragma unroll
      for (int i = 0; i < FPW / 4; ++i) {
        const float4 s4 = *reinterpret_cast<const float4*>(pg + PG::OFF_KS + 4 * (cw + 4 * i));
        const float4 z4 = *reinterpret_cast<const float4*>(pg + PG::OFF_KZ + 4 * (cw + 4 * i));
        sv[4 * i] = s4.x; sv[4 * i + 1] = s4.y; sv[4 * i + 2] = s4.z; sv[4 * i + 3] = s4.w;
        zv[4 * i] = z4.x; zv[4 * i + 1] = z4.y; zv[4 * i + 2] = z4.z; zv[4 * i + 3] = z4.w;
      }
      if (ek) {
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
          sv[i] = ldexpf(sv[i], -ek);
          zv[i] = ldexpf(zv[i], -ek);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float x[FPW];
        codes_f32(kp[mt][w], x);
#pragma unroll
        for (int i = 0; i < FPW; ++i) x[i] = fmaf(x[i], sv[i], zv[i]);
        // k-steps of this word: 8 channels each, fragment order {0,2,1,3,4,6,5,7}
#pragma unroll
        for (int k8 = 0; k8 < FPW / 8; ++k8) {
          const float* y = x + 8 * k8;
          uint32_t hi[4], lo[4];
          split_f16(y[0], y[2], hi[0], lo[0]);
          split_f16(y[1], y[3], hi[1], lo[1]);
          split_f16(y[4], y[6], hi[2], lo[2]);
          split_f16(y[5], y[7], hi[3], lo[3]);
          const half8 ah = cat4h(hi[0], hi[1], hi[2], hi[3]), al = cat4h(lo[0], lo[1], lo[2], lo[3]);
          const int ks = w * (FPW / 8) + k8;
          c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bqh[ks], c[mt], 0, 0, 0);
          c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bqh[ks], c[mt], 0, 0, 0);
          c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bql[ks], c[mt], 0, 0, 0);
        }
      }
    }
    float s[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * mt + r] = c[mt][r];
    const int es = ek + eq;
    if (es) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = ldexpf(s[i], es);
    }
    // causal mask: a page that the first query does not see whole (its last
    // page, or one past it when a later query's token opens it)
    const bool masked_page = Tb - t0 < kPage;
    const int nvalid = static_cast<int>(Tj - t0);
    if (masked_page) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile_tok<false>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = -INFINITY;
    }
    softmax_update(s, std::integral_constant<int, 8>{});
    if (masked_page) {   // a column with no token yet has max -inf: weight 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile_tok<false>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = 0.f;
    }
    // per-token value scale and offset of this lane's tokens tile_tok(mt, 4g + r)
    const float4 vs0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + 32 * g);
    const float4 vs1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + 16 + 32 * g);
    const float4 vz0 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + 32 * g);
    const float4 vz1 = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + 16 + 32 * g);
    const float vsv[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    const float vzv[8] = {vz0.x, vz0.y, vz0.z, vz0.w, vz1.x, vz1.y, vz1.z, vz1.w};
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      l_lane += s[i];
      z_lane = fmaf(s[i], vzv[i], z_lane);
      pv[i] = s[i] * vsv[i];
    }
    // P' rows (pair j) in bf16 high and remainder parts, tokens in the order
    // {0,2,1,3,4,6,5,7}: two A operands on the same value codes
    uint32_t ph[4], pl[4];
    split_bf16(pv[0], pv[2], ph[0], pl[0]);
    split_bf16(pv[1], pv[3], ph[1], pl[1]);
    split_bf16(pv[4], pv[6], ph[2], pl[2]);
    split_bf16(pv[5], pv[7], ph[3], pl[3]);
    const bf16x8 aph = __builtin_bit_cast(bf16x8, uint4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 apl = __builtin_bit_cast(bf16x8, uint4{pl[0], pl[1], pl[2], pl[3]});
    if constexpr (VB == 4) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {   // a word per channel tile: tokens 8g..8g+7
        const uint32_t w = *reinterpret_cast<const uint32_t*>(pg + PG::OFF_VC + (16 * nt + j) * VROW + 4 * g);
        const uint32_t y0 = w & 0x0F0F0F0Fu, y1 = (w >> 4) & 0x0F0F0F0Fu;
        const bf16x8 bw = __builtin_bit_cast(bf16x8, uint4{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, false)),
                                                           bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, false)),
                                                           bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y0, 512.0f, true)),
                                                           bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y1, 512.0f, true))});
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aph, bw, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apl, bw, acc[nt], 0, 0, 0);
      }
    } else {
#pragma unroll
    for (int nt = 0; nt < NT; nt += 2) {   // two channel tiles per code word
      const uint8_t* col = pg + PG::OFF_VC + (16 * nt + j) * VROW + 2 * g;
      u16x2 xv;
      xv.x = *reinterpret_cast<const uint16_t*>(col);
      xv.y = *reinterpret_cast<const uint16_t*>(col + 16 * VROW);
      const uint32_t x = __builtin_bit_cast(uint32_t, xv);
      const uint32_t y0 = x & 0x33333333u, y1 = (x >> 2) & 0x33333333u;
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, uint4{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 0)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 0)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 1)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 1))});
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, uint4{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 2)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 2)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 3)),
                                                         bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 3))});
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aph, b0, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apl, b0, acc[nt], 0, 0, 0);
      acc[nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aph, b1, acc[nt + 1], 0, 0, 0);
      acc[nt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apl, b1, acc[nt + 1], 0, 0, 0);
    }
    }
  };

  // ---- residual (unquantised) tokens, 8 per step -----------------------------
  uint8_t* wring = wbuf + PG::BYTES;
  constexpr int LPR = 2 * D / 16;           // lanes per bf16 row
  constexpr int RPI = 64 / LPR;             // rows per 16-byte-per-lane copy
  constexpr int RSTEP = 8;
  auto issue_step = [&](int hs) -> int {    // returns the copies issued
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    const int nv = static_cast<int>(TbL - t0 < RSTEP ? TbL - t0 : RSTEP);
    const int row_in = lane / LPR, col_b = (lane % LPR) * 16;
    const int slots = static_cast<int>(p.ring_slots);
    const int slot0 = static_cast<int>(t0 % p.ring_slots);
    int issued = 0;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
      for (int i = 0; i < (RSTEP + RPI - 1) / RPI; ++i) {
        if (i * RPI >= nv) continue;          // wave-uniform
        const int r = i * RPI + row_in;
        const int slot = slot0 + r < slots ? slot0 + r : slot0 + r - slots;
        const uint8_t* src = ringp + (kv * p.ring_slots + slot) * (2 * D) + col_b;
        if (r < nv && r < RSTEP) dma16(src, lds_addr(wring + kv * RSTEP * 2 * D + i * 1024));
        ++issued;
      }
    }
    // value rows of absent tokens must be finite (they meet weight 0): zero them
    for (int i = lane; i < (RSTEP - nv) * 2 * D / 16; i += 64)
      *reinterpret_cast<uint4*>(wring + RSTEP * 2 * D + nv * 2 * D + i * 16) = uint4{0u, 0u, 0u, 0u};
    return issued;
  };
  // B operands of the residual key product: q' of pair j (unscaled) in three
  // bf16 parts (high, middle, remainder), channels 32 ks + 8 g + 0..7
  auto qpart = [&](int part, int ks) -> bf16x8 {
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 qq = *reinterpret_cast<const float2*>(&qs[j][32 * ks + 8 * g + 2 * i]);
      const float h0 = bf16_trunc(qq.x), h1 = bf16_trunc(qq.y);
      const float m0 = bf16_trunc(qq.x - h0), m1 = bf16_trunc(qq.y - h1);
      const float x0 = part == 0 ? h0 : (part == 1 ? m0 : qq.x - h0 - m0);
      const float x1 = part == 0 ? h1 : (part == 1 ? m1 : qq.y - h1 - m1);
      w4[i] = pack_bf16(x0, x1);
    }
    return __builtin_bit_cast(bf16x8, uint4{w4[0], w4[1], w4[2], w4[3]});
  };
  // tile rows 8..15 of a step repeat rows 0..7 and are masked
  auto process_step = [&](int hs) {
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    const int nv = static_cast<int>(Tj - t0 < RSTEP ? Tj - t0 : RSTEP);
    floatx4 cr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wring + (j & 7) * 2 * D + (32 * ks + 8 * g) * 2);
#pragma unroll
      for (int part = 0; part < 3; ++part)
        cr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qpart(part, ks), cr, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (4 * g + r < nv) ? cr[r] : -INFINITY;
    softmax_update(sc, std::integral_constant<int, 4>{});
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = 4 * g + r < nv ? sc[r] : 0.f;   // absent tokens: weight 0
#pragma unroll
    for (int r = 0; r < 4; ++r) l_lane += sc[r];
    uint32_t ph[2], pl[2];
    split_bf16(sc[0], sc[1], ph[0], pl[0]);
    split_bf16(sc[2], sc[3], ph[1], pl[1]);
    const bf16x8 aph = __builtin_bit_cast(bf16x8, uint4{ph[0], ph[1], 0u, 0u});
    const bf16x8 apl = __builtin_bit_cast(bf16x8, uint4{pl[0], pl[1], 0u, 0u});
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int c = 16 * nt + j;
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(wring + RSTEP * 2 * D) + c;
      const int t4 = (4 * g) & 7;             // tokens >= 8 carry weight 0
      const uint32_t v0 = vr[(t4 + 0) * D], v1 = vr[(t4 + 1) * D];
      const uint32_t v2 = vr[(t4 + 2) * D], v3 = vr[(t4 + 3) * D];
      const bf16x8 bv = __builtin_bit_cast(bf16x8, uint4{v0 | (v1 << 16), v2 | (v3 << 16), 0u, 0u});
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aph, bv, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apl, bv, acc[nt], 0, 0, 0);
    }
  };

  // ---- first requests: q (wave 0), this wave's first residual step, its first page
  const int my_wave = (NW - 1 - wave) * p.splits + split;
  const int q_bytes = HG * D * (p.q_bf16 ? 2 : 4);   // one query's heads of this KV head
  int after_q = 0;
  if (wave == 0) {
#pragma unroll
    for (int qq = 0; qq < QN; ++qq) {
      const uint8_t* qsrc = p.q + (static_cast<int64_t>(b * p.nq + qi + qq) * p.q_heads + h * HG) * D * (p.q_bf16 ? 2 : 4);
      for (int off = 0; off < q_bytes; off += 1024)
        if (off + lane * 16 < q_bytes) dma16(qsrc + off + lane * 16, lds_addr(&qs[0][0]) + qq * q_bytes + off);
    }
  }
  const bool has_step = my_wave < n_steps;
  if (has_step) after_q += issue_step(my_wave);
  if (n_mine > 0) {
    issue_page(0);
    after_q += PG::DMA;
  }
  if (wave == 0) wait_vm_upto(after_q);   // q has landed
  __syncthreads();
  {
    // raw query (bf16 or f32) -> f32 * sm_scale * log2(e), in place
    constexpr int PER = (GC * D + NTH - 1) / NTH;
    float qv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      qv[k] = 0.f;
      if (i < GC * D)
        qv[k] = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(&qs[0][0])[i]) : (&qs[0][0])[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      if (i < GC * D) (&qs[0][0])[i] = qv[k] * p.qscale;
    }
    __syncthreads();
  }
  {
    // the key product's B operand: q' of pair j, channels g CPG + 8 ks +
    // {0,2,1,3,4,6,5,7}, scaled below 2^15 (the wave sees every pair and channel)
    float qa = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) qa = fmaxf(qa, fabsf(qs[j][g * CPG + 8 * ks + i]));
    if (__builtin_amdgcn_ballot_w64(qa >= 32768.f) != 0) {
      int ex;
      frexpf(wave_max(qa), &ex);
      eq = __builtin_amdgcn_readfirstlane(ex - 15);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ldexpf(qs[j][g * CPG + 8 * ks + i], -eq);
      uint32_t hi[4], lo[4];
      split_f16(y[0], y[2], hi[0], lo[0]);
      split_f16(y[1], y[3], hi[1], lo[1]);
      split_f16(y[4], y[6], hi[2], lo[2]);
      split_f16(y[5], y[7], hi[3], lo[3]);
      bqh[ks] = cat4h(hi[0], hi[1], hi[2], hi[3]);
      bql[ks] = cat4h(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  if (has_step) {
    if (n_mine > 0) wait_vm<PG::DMA>();   // the first page may stay in flight
    else wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    process_step(my_wave);
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  }

  // ---- pages: DMA pipeline, one page ahead (page 0 already requested) --------
#pragma unroll 1
  for (int k = 0; k < n_mine; ++k) {
    wait_lds();   // the buffer about to be refilled has been read
    __builtin_amdgcn_wave_barrier();
    const bool next = k + 1 < n_mine;
    if (next) issue_page(k + 1);
    if (next) wait_vm<PG::DMA>();
    else wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    process_page(wbuf + (k % 2) * PG::BYTES, static_cast<int64_t>(pg0 + wave + NW * k) * kPage);
  }

  // ---- any further residual steps of this wave ---------------------------------
#pragma unroll 1
  for (int hs = my_wave + waves_total; hs < n_steps; hs += waves_total) {
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    issue_step(hs);
    wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    process_step(hs);
  }
  wait_lds();

  // ---- wave epilogue: column j's sums over the lane groups ----------------------
  float lsum[GC], zsum[GC], mh[GC];
  {
    float l_ = l_lane, z_ = z_lane;
    l_ += xor16(l_);
    l_ += xor32(l_);
    z_ += xor16(z_);
    z_ += xor32(z_);
#pragma unroll
    for (int vh = 0; vh < GC; ++vh) {
      lsum[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_), vh));
      zsum[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z_), vh));
      mh[vh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_lane), vh));
    }
  }
  finish_unit<D, HG, NW, QN, true>(p, acc, mh, lsum, zsum, arena, last_block, b, qi, h, split);
}

// ---- long chunks of queries: one pass over the pages for 32 queries ----------
// 32 consecutive queries of a sequence per block (GQA 4, head_dim 128, 2- or
// 4-bit keys, 2-bit values), wave w taking queries 4w..4w+3 (its 16 (query,
// head) pairs are the columns of its key product, as in kivi_deq_kernel).
// The block walks the tokens in chunks of 32: the quantised pages up to the
// last query's, then the residual ring up to its token. Each chunk is copied
// to LDS once, and the block dequantises it once: wave w builds the f16
// high/remainder key fragment (token tile w / 4, k-step w % 4) and the bf16
// value fragment of channel tile w for every wave to read. Every wave then
// takes the whole chunk against its own queries. Per chunk: copy (issued
// during the previous chunk's products), barrier, dequantisation, barrier,
// products. One split: the grid's rows are (sequence, 32 queries), enough to
// fill the chip when batch * KV heads * n_q / 32 >= 256, and each wave writes
// its own rows' outputs.
template <int KB>
__device__ __forceinline__ void key_codes8(uint32_t wd, int half, float* x) {
  // the 8 codes of k-step `half` of a word (2-bit: fields 8 half ..; 4-bit:
  // the word), field order
  if constexpr (KB == 2) {
    const uint32_t y0 = wd & 0x33333333u, y1 = (wd >> 2) & 0x33333333u;
    float2 a0, a1, a2, a3;
    if (half == 0) {
      a0 = codes2_f32<0>(y0); a1 = codes2_f32<0>(y1); a2 = codes2_f32<1>(y0); a3 = codes2_f32<1>(y1);
    } else {
      a0 = codes2_f32<2>(y0); a1 = codes2_f32<2>(y1); a2 = codes2_f32<3>(y0); a3 = codes2_f32<3>(y1);
    }
    x[0] = a0.x; x[2] = a0.y; x[1] = a1.x; x[3] = a1.y;
    x[4] = a2.x; x[6] = a2.y; x[5] = a3.x; x[7] = a3.y;
  } else {
    const uint32_t y0 = wd & 0x0F0F0F0Fu, y1 = (wd >> 4) & 0x0F0F0F0Fu;
    const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y0, 512.0f, false);
    const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y1, 512.0f, false);
    const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y0, 512.0f, true);
    const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(y1, 512.0f, true);
    x[0] = a0[0]; x[2] = a0[1]; x[1] = a1[0]; x[3] = a1[1];
    x[4] = a2[0]; x[6] = a2[1]; x[5] = a3[0]; x[7] = a3[1];
  }
}

template <int KB>
__global__ __launch_bounds__(512, 1) void kivi_chunk_kernel(MfmaParams p) {
  constexpr int D = 128, VB = 2, HG = 4;
  constexpr int NW = 8, NTH = 512, QB = 4 * NW;   // 32 queries per block
  using PG = PageGeom<KB, VB, D>;
  constexpr int KS = D / 32, NT = D / 16, CPG = D / 4;
  constexpr int KROW = D * KB / 8, CPR_K = KROW / 16;
  constexpr int FPW = 32 / KB, KW = CPG / FPW;
  constexpr int VROW = 32 * VB / 8;
  constexpr int ROWB = 2 * D;                      // bytes of a bf16 residual row
  constexpr int STAGE = 2 * kPage * ROWB;          // a ring chunk: 32 key + 32 value rows
  static_assert(PG::BYTES <= STAGE && NW == 2 * KS && NW == NT, "one fragment of each kind per wave");
  constexpr float kLevels = float((1 << KB) - 1);
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][STAGE];
  __shared__ __attribute__((aligned(16))) uint4 kfrag[2 * KS][2][64];   // [tile * KS + ks][hi, lo][lane]
  __shared__ __attribute__((aligned(16))) uint4 vfrag[NT][64];          // [channel tile][lane]
  __shared__ __attribute__((aligned(16))) float vsc[kPage], vzc[kPage];
  __shared__ int chunk_e;                                               // the chunk's key scaling

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int h = blockIdx.y;
  const int groups = p.nq / QB;
  const int b = blockIdx.z / groups, qi = (blockIdx.z - b * groups) * QB;
  const uint8_t* ringp = p.pm.ring(b, h);
  const int64_t q_tokens = p.q_tokens;
  const int64_t Tb = p.T - (p.nq - 1 - qi);        // tokens the block's first query sees
  const int64_t TbL = Tb + QB - 1;                 // ... and its last
  const int64_t Tj = Tb + 4 * wave + j / HG;       // ... and column j of this wave
  const int n_pages = static_cast<int>(TbL <= q_tokens ? (TbL + kPage - 1) / kPage : q_tokens / kPage);
  const int n_ring = TbL <= q_tokens ? 0 : static_cast<int>((TbL - q_tokens + kPage - 1) / kPage);
  const int n_chunks = n_pages + n_ring;

  // stale ring rows (past the last query's token) must be finite: zero both stages
  for (int i = tid; i < 2 * STAGE / 16; i += NTH) reinterpret_cast<uint4*>(&stage[0][0])[i] = uint4{0u, 0u, 0u, 0u};
  __syncthreads();   // zeroed before any copy lands

  // ---- the key product's B operand for this wave's 16 pairs (q' scaled by 2^-eq)
  half8 bqh[KS], bql[KS];
  int eq = 0;
  {
    const int64_t row = static_cast<int64_t>(b) * p.nq + qi + 4 * wave + j / HG;
    const int64_t base = (row * p.q_heads + h * HG + j % HG) * D;
    float y[KS][8];
    float qa = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = g * CPG + 8 * ks;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y[ks][i] = load_q(p.q, base + c0 + i, p.q_bf16) * p.qscale;
        qa = fmaxf(qa, fabsf(y[ks][i]));
      }
    }
    if (__builtin_amdgcn_ballot_w64(qa >= 32768.f) != 0) {
      int ex;
      frexpf(wave_max(qa), &ex);
      eq = __builtin_amdgcn_readfirstlane(ex - 15);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float z[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = ldexpf(y[ks][i], -eq);
      uint32_t hi[4], lo[4];
      split_f16(z[0], z[2], hi[0], lo[0]);
      split_f16(z[1], z[3], hi[1], lo[1]);
      split_f16(z[4], z[6], hi[2], lo[2]);
      split_f16(z[5], z[7], hi[3], lo[3]);
      bqh[ks] = cat4h(hi[0], hi[1], hi[2], hi[3]);
      bql[ks] = cat4h(lo[0], lo[1], lo[2], lo[3]);
    }
  }

  floatx4 acc[NT];   // rows 4g + r: pair 4g + r of this wave
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_lane = -INFINITY, l_lane = 0.f, z_lane = 0.f;

  // chunk c: page c (c < n_pages), else ring tokens from q_tokens + 32 (c - n_pages)
  auto issue_chunk = [&](int c) {
    uint8_t* dst = stage[c & 1];
    if (c < n_pages) {
      const uint8_t* src = p.pm.page(b, h, c);
      const int off = wave * 1024 + lane * 16;
      int from = off;
      if (off < PG::CODES) from = krow_off<CPR_K>(off / KROW, off % KROW);
      if (wave * 1024 < PG::BYTES && off < PG::BYTES) dma16(src + from, lds_addr(dst + wave * 1024));
    } else {
      const int64_t t0 = q_tokens + static_cast<int64_t>(c - n_pages) * kPage;
      const int r = wave * 4 + lane / 16, cb = (lane % 16) * 16;   // row r of the chunk, 16 bytes
      const bool valid = t0 + r < TbL;
      const int64_t slot = (t0 + r) % p.ring_slots;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        uint8_t* d = dst + kv * kPage * ROWB;
        if (valid) dma16(ringp + (kv * p.ring_slots + slot) * ROWB + cb, lds_addr(d + wave * 1024));
        else *reinterpret_cast<uint4*>(d + r * ROWB + cb) = uint4{0u, 0u, 0u, 0u};
      }
    }
  };

  // wave w's fragments of chunk c (token tile w / KS, k-step w % KS; channel tile w)
  auto dequant_chunk = [&](int c) {
    const uint8_t* st = stage[c & 1];
    const int mt = wave / KS, ks = wave % KS;
    const int tok = tile_tok<false>(mt, j);
    const int c0 = g * CPG + 8 * ks;
    float x[8];
    int e = 0;
    if (c < n_pages) {
      // page bound max(|z|, |z + levels s|) over the channels (every wave the same)
      float kb = 0.f;
#pragma unroll
      for (int cc = lane; cc < D; cc += 64) {
        const float sc = reinterpret_cast<const float*>(st + PG::OFF_KS)[cc];
        const float zc = reinterpret_cast<const float*>(st + PG::OFF_KZ)[cc];
        kb = fmaxf(kb, fmaxf(fabsf(zc), fabsf(fmaf(kLevels, sc, zc))));
      }
      if (__builtin_amdgcn_ballot_w64(kb >= 32768.f) != 0) {
        int ex;
        frexpf(wave_max(kb), &ex);
        e = __builtin_amdgcn_readfirstlane(ex - 15);
      }
      const int word = (8 * ks) / FPW;
      const uint32_t wd = *reinterpret_cast<const uint32_t*>(st + krow_off<CPR_K>(tok, g * (KW * 4) + 4 * word));
      key_codes8<KB>(wd, ((8 * ks) % FPW) / 8, x);
      const float4 s0 = *reinterpret_cast<const float4*>(st + PG::OFF_KS + 4 * c0);
      const float4 s1 = *reinterpret_cast<const float4*>(st + PG::OFF_KS + 4 * c0 + 16);
      const float4 z0 = *reinterpret_cast<const float4*>(st + PG::OFF_KZ + 4 * c0);
      const float4 z1 = *reinterpret_cast<const float4*>(st + PG::OFF_KZ + 4 * c0 + 16);
      float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      if (e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sv[i] = ldexpf(sv[i], -e);
          zv[i] = ldexpf(zv[i], -e);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], sv[i], zv[i]);
      // values: channel tile `wave`, tokens 8g .. 8g + 7
      const uint32_t xv = *reinterpret_cast<const uint16_t*>(st + PG::OFF_VC + (16 * wave + j) * VROW + 2 * g);
      const uint32_t y0 = xv & 0x3333u, y1 = (xv >> 2) & 0x3333u;
      vfrag[wave][lane] = uint4{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 0)),
                                bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 0)),
                                bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 1)),
                                bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 1))};
      if (wave == 0 && lane < kPage) {
        vsc[lane] = reinterpret_cast<const float*>(st + PG::OFF_VS)[lane];
        vzc[lane] = reinterpret_cast<const float*>(st + PG::OFF_VZ)[lane];
      }
    } else {
      // ring rows: bound max |k| over the chunk (every wave the same)
      float kb = 0.f;
#pragma unroll
      for (int i = 0; i < kPage * ROWB / (64 * 16); ++i) {
        float f[8];
        unpack_bf16x8(reinterpret_cast<const uint4*>(st)[i * 64 + lane], f);
#pragma unroll
        for (int k = 0; k < 8; ++k) kb = fmaxf(kb, fabsf(f[k]));
      }
      if (__builtin_amdgcn_ballot_w64(kb >= 32768.f) != 0) {
        int ex;
        frexpf(wave_max(kb), &ex);
        e = __builtin_amdgcn_readfirstlane(ex - 15);
      }
      unpack_bf16x8(*reinterpret_cast<const uint4*>(st + tok * ROWB + 2 * c0), x);
      if (e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = ldexpf(x[i], -e);
      }
      // values: channel 16 wave + j of tokens 8g + {0,2,1,3,4,6,5,7}
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(st + kPage * ROWB) + 16 * wave + j;
      uint32_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = vr[(8 * g + i) * D];
      vfrag[wave][lane] = uint4{v[0] | (v[2] << 16), v[1] | (v[3] << 16), v[4] | (v[6] << 16), v[5] | (v[7] << 16)};
      if (wave == 0 && lane < kPage) {
        vsc[lane] = 1.f;
        vzc[lane] = 0.f;
      }
    }
    if (wave == 0 && lane == 0) chunk_e = e;
    uint32_t hi[4], lo[4];
    split_f16(x[0], x[2], hi[0], lo[0]);
    split_f16(x[1], x[3], hi[1], lo[1]);
    split_f16(x[4], x[6], hi[2], lo[2]);
    split_f16(x[5], x[7], hi[3], lo[3]);
    kfrag[wave][0][lane] = uint4{hi[0], hi[1], hi[2], hi[3]};
    kfrag[wave][1][lane] = uint4{lo[0], lo[1], lo[2], lo[3]};
  };

  auto compute_chunk = [&](int c) {
    const int64_t t0 = c < n_pages ? static_cast<int64_t>(c) * kPage
                                   : q_tokens + static_cast<int64_t>(c - n_pages) * kPage;
    floatx4 sc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 fh = kfrag[mt * KS + ks][0][lane], fl = kfrag[mt * KS + ks][1][lane];
        const half8 ah = cat4h(fh.x, fh.y, fh.z, fh.w), al = cat4h(fl.x, fl.y, fl.z, fl.w);
        sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bqh[ks], sc[mt], 0, 0, 0);
        sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bqh[ks], sc[mt], 0, 0, 0);
        sc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bql[ks], sc[mt], 0, 0, 0);
      }
    float s[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[4 * mt + r] = sc[mt][r];
    const int es = chunk_e + eq;
    if (es) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = ldexpf(s[i], es);
    }
    // tokens past each column's query (and stale ring rows) are masked
    const bool masked = Tb - t0 < kPage;
    const int nvalid = static_cast<int>(Tj - t0);
    if (masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile_tok<false>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = -INFINITY;
    }
    float pmax = s[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) pmax = fmaxf(pmax, s[i]);
    if (__builtin_amdgcn_ballot_w64(pmax > m_lane + kMaxSlack) != 0) {
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      const float m_new = fmaxf(m_lane, pmax);
      const float alpha = m_new == m_lane ? 1.0f : fast_exp2(m_lane - m_new);
      l_lane *= alpha;
      z_lane *= alpha;
      m_lane = m_new;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= a;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = fast_exp2(s[i] - m_lane);
    if (masked) {   // a column with no token yet has max -inf: weight 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile_tok<false>(mt, 4 * g + r) >= nvalid) s[4 * mt + r] = 0.f;
    }
    const float4 vs0 = *reinterpret_cast<const float4*>(&vsc[8 * g]);
    const float4 vs1 = *reinterpret_cast<const float4*>(&vsc[8 * g + 4]);
    const float4 vz0 = *reinterpret_cast<const float4*>(&vzc[8 * g]);
    const float4 vz1 = *reinterpret_cast<const float4*>(&vzc[8 * g + 4]);
    const float vsv[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
    const float vzv[8] = {vz0.x, vz0.y, vz0.z, vz0.w, vz1.x, vz1.y, vz1.z, vz1.w};
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      l_lane += s[i];
      z_lane = fmaf(s[i], vzv[i], z_lane);
      pv[i] = s[i] * vsv[i];
    }
    uint32_t ph[4], pl[4];
    split_bf16(pv[0], pv[2], ph[0], pl[0]);
    split_bf16(pv[1], pv[3], ph[1], pl[1]);
    split_bf16(pv[4], pv[6], ph[2], pl[2]);
    split_bf16(pv[5], pv[7], ph[3], pl[3]);
    const bf16x8 aph = __builtin_bit_cast(bf16x8, uint4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 apl = __builtin_bit_cast(bf16x8, uint4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, vfrag[nt][lane]);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aph, bv, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apl, bv, acc[nt], 0, 0, 0);
    }
  };

  if (n_chunks > 0) issue_chunk(0);
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    wait_vm<0>();      // this wave's copies of chunk c have landed
    __syncthreads();   // chunk c is in its stage; every wave is done with chunk c - 1's fragments
    dequant_chunk(c);
    __syncthreads();   // the fragments of chunk c are complete
    if (c + 1 < n_chunks) issue_chunk(c + 1);
    compute_chunk(c);
  }

  // ---- outputs of this wave's 16 pairs: (acc + sum p z) / sum p -----------------
  float l_ = l_lane, z_ = z_lane;
  l_ += xor16(l_);
  l_ += xor32(l_);
  z_ += xor16(z_);
  z_ += xor32(z_);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int vh = 4 * g + r;   // this lane's accumulator rows
    const float lv = __shfl(l_, vh, 64), zv = __shfl(z_, vh, 64);
    const int64_t row = static_cast<int64_t>(b) * p.nq + qi + 4 * wave + vh / HG;
    float* o = p.out + (row * p.q_heads + h * HG + vh % HG) * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[16 * nt + j] = (acc[nt][r] + zv) / lv;
  }
}

// ---- rotary keys, GQA group of 4: dense scores on v_mfma_f32_4x4x1_16b_f32 ----
// Same result as kivi_mfma_kernel<2, D, 4, true> with the key product laid out
// so that no MFMA column is wasted. Lane l takes token l % 32 of a page (or of
// a residual step) and the channel half l / 32; the 16 blocks of the 4x4x1
// instruction are (token quad, channel half) and its 4 columns the 4 heads, so
// one instruction is one channel of 32 tokens x 4 heads for each half:
//   A = R(omega j) (code * s + z) of the lane's token j and channel (fp32),
//   B = qpage of the lane's head l % 4 and channel, qpage = R(omega (T-1-t0)) q.
// The two halves are added across lanes (l, l ^ 32). Every lane then holds the
// scores of tokens 4((l/4) % 8) + r of head l % 4, the running max of each head
// is wave-uniform, and the weights P' are moved through LDS into the operand
// layout of the value product (v_mfma_f32_16x16x32_bf16, as in
// kivi_mfma_kernel).
// The rotation of token position j by omega_i is a block-wide LDS table
// (every wave uses the same token-to-lane map), so it costs no registers; the
// key product runs in two chunks of a quarter of the channels to keep fewer
// dequantised keys live. With 4 waves per block, LDS (53 760 B at d = 128)
// and registers fit three blocks per CU.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 3) void rope4_kernel(MfmaParams p) {
  constexpr int HG = 4, BITS = 2;
  constexpr int NTH = NW * 64;           // threads of the block
  using PG = PageGeom<BITS, BITS, D>;
  constexpr int NT = D / 16;             // channel tiles of the value product
  constexpr int KROW = D * BITS / 8;     // bytes per key token row
  constexpr int CPR_K = KROW / 16;
  constexpr int HALF = D / 2;            // channels per lane
  constexpr int NPL = HALF / 2;          // channel pairs per lane
  constexpr int CH = HALF / 2;           // channels per chunk of the key product
  constexpr int VROW = 32 * BITS / 8;    // bytes per value channel column
  constexpr int RSTEP = 8;
  static_assert(CH % 16 == 0, "whole code words per chunk");
  // Per-wave LDS: two page buffers. A residual step (8 key + 8 value rows)
  // borrows them: a wave takes all its steps before it requests its first page.
  constexpr int WAVE_LDS = 2 * PG::BYTES;
  static_assert(WAVE_LDS >= PG::RING, "a residual step fits the page buffers");
  constexpr int RED = NW * HG * (D + 2) * 4;
  constexpr int ARENA = NW * WAVE_LDS > RED + 16 ? NW * WAVE_LDS : RED + 16;

  // qpage rows (head, channel half) padded by 16 bytes: the 8 rows that the
  // lanes of a wave read together start in different LDS banks
  constexpr int QROW = HALF + 4;
  __shared__ __attribute__((aligned(16))) float qpage[NW][HG * 2][QROW];
  // weights P' of the page in hand, [hi/lo][head][32 tokens] in bf16, in the
  // k order of the value operand
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[NW][2][HG][32];
  __shared__ __attribute__((aligned(16))) uint8_t arena[ARENA];
  // rotation table: entry (half, m2, token) = {cos, sin} of omega_i * token for
  // the pairs i = half * NPL + 2 m2 and the next one; consecutive tokens are
  // consecutive 16-byte entries (the 32 lanes of a half read 512 bytes)
  __shared__ __attribute__((aligned(16))) float4 rtab[2 * (NPL / 2) * 32];
  // set-up data in LDS that is idle at that time: the scaled query in the
  // rotation table (read into registers before the table is built), omega_i /
  // (2 pi) in wave 0's weight buffer (each lane keeps its own in a register);
  // the last-block flag of the merge lives in the arena, which is free then
  static_assert(HG * D * 4 <= static_cast<int>(sizeof(rtab)), "query fits the table");
  static_assert(D / 2 * 8 <= static_cast<int>(sizeof(pbuf)), "omega fits the weight buffers");
  float (*qs)[D] = reinterpret_cast<float (*)[D]>(&rtab[0]);
  double* w2pi = reinterpret_cast<double*>(&pbuf[0][0][0][0]);
  int& last_block = *reinterpret_cast<int*>(arena + ARENA - 16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform in the wave
  const int j = lane & 15, g = lane >> 4;          // 16x16 operand coordinates
  const int hd = lane & 3;                          // head of this lane (4x4 column)
  const int tk = lane & 31;                         // token of this lane (4x4 row)
  const int hf = lane >> 5;                         // channel half of this lane
  const int split = blockIdx.x, h = blockIdx.y;
  const int b = blockIdx.z / p.nq, qi = blockIdx.z - b * p.nq;   // sequence, its query
  const uint8_t* ringp = p.pm.ring(b, h);
  uint8_t* wbuf = arena + wave * WAVE_LDS;
  uint8_t* wring = wbuf;
  // tokens this sequence holds (a ragged batch: its own fill level, and its
  // own split between quantised pages and the ring)
  const int64_t fill = seq_len(p.seq_tokens, b, p.T);
  int64_t q_tokens = p.q_tokens;
  int32_t n_pages = p.n_pages, n_steps = p.n_steps;
  if (p.seq_tokens) {
    q_tokens = kivi_quantised(fill, p.residual);
    n_pages = static_cast<int32_t>(q_tokens / kPage);
  }
  // query qi of nq: position fill - nq + qi (as above)
  const int64_t Tb = fill - (p.nq - 1 - qi);
  if (p.seq_tokens || p.nq > 1) n_steps = static_cast<int32_t>((Tb - q_tokens + 7) / 8);
  const bool in_page = Tb <= q_tokens;   // block-uniform: mask this row's last page
  if (in_page) {
    n_pages = static_cast<int32_t>((Tb + kPage - 1) / kPage);
    n_steps = 0;
  }

  const int pg0 = static_cast<int>(static_cast<int64_t>(split) * n_pages / p.splits);
  const int pg1 = static_cast<int>(static_cast<int64_t>(split + 1) * n_pages / p.splits);
  const int n_mine = pg0 + wave < pg1 ? (pg1 - pg0 - wave + NW - 1) / NW : 0;
  const int waves_total = p.splits * NW;
  const int my_wave = (NW - 1 - wave) * p.splits + split;

  auto issue_page = [&](int k) {
    const uint8_t* src = p.pm.page(b, h, pg0 + wave + NW * k);
    const uint32_t dst = lds_addr(wbuf + (k % 2) * PG::BYTES);
#pragma unroll
    for (int i = 0; i < PG::DMA; ++i) {
      const int off = i * 1024 + lane * 16;
      int from = off;
      if (off < PG::CODES) from = krow_off<CPR_K>(off / KROW, off % KROW);
      if (i + 1 < PG::DMA || off < PG::BYTES) dma16(src + from, dst + i * 1024);
    }
  };
  constexpr int LPR = 2 * D / 16;
  constexpr int RPI = 64 / LPR;
  auto issue_step = [&](int hs) -> int {
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    const int nv = static_cast<int>(Tb - t0 < RSTEP ? Tb - t0 : RSTEP);
    const int row_in = lane / LPR, col_b = (lane % LPR) * 16;
    const int slots = static_cast<int>(p.ring_slots);
    const int slot0 = static_cast<int>(t0 % p.ring_slots);
    int issued = 0;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
#pragma unroll
      for (int i = 0; i < (RSTEP + RPI - 1) / RPI; ++i) {
        if (i * RPI >= nv) continue;
        const int r = i * RPI + row_in;
        const int slot = slot0 + r < slots ? slot0 + r : slot0 + r - slots;
        const uint8_t* src = ringp + (kv * p.ring_slots + slot) * (2 * D) + col_b;
        if (r < nv && r < RSTEP) dma16(src, lds_addr(wring + kv * RSTEP * 2 * D + i * 1024));
        ++issued;
      }
    }
    for (int i = lane; i < (RSTEP - nv) * 2 * D / 16; i += 64)
      *reinterpret_cast<uint4*>(wring + RSTEP * 2 * D + nv * 2 * D + i * 16) = uint4{0u, 0u, 0u, 0u};
    return issued;
  };

  // ---- first requests: q (wave 0), this wave's first residual step or page ----
  const int q_bytes = HG * D * (p.q_bf16 ? 2 : 4);
  int after_q = 0;
  if (wave == 0) {
    const uint8_t* qsrc = p.q + (static_cast<int64_t>(b * p.nq + qi) * p.q_heads + h * HG) * D * (p.q_bf16 ? 2 : 4);
    for (int off = 0; off < q_bytes; off += 1024)
      if (off + lane * 16 < q_bytes) dma16(qsrc + off + lane * 16, lds_addr(&qs[0][0]) + off);
  }
  const bool has_step = my_wave < n_steps;
  if (has_step) {
    after_q += issue_step(my_wave);
  } else if (n_mine > 0) {
    issue_page(0);
    after_q += PG::DMA;
  }
  for (int i = tid; i < D / 2; i += NTH)
    w2pi[i] = pow(p.rope_theta, -2.0 * i / D) * 0.15915494309189535;   // omega_i / (2 pi)
  if (wave == 0) wait_vm_upto(after_q);   // q has landed
  __syncthreads();
  {
    constexpr int PER = (HG * D + NTH - 1) / NTH;
    float qv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      qv[k] = 0.f;
      if (i < HG * D)
        qv[k] = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(&qs[0][0])[i])
                         : (&qs[0][0])[i];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NTH;
      if (i < HG * D) (&qs[0][0])[i] = qv[k] * p.qscale;
    }
  }
  __syncthreads();
  float qpair[HG][2];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    qpair[hh][0] = lane < D / 2 ? qs[hh][2 * lane] : 0.f;
    qpair[hh][1] = lane < D / 2 ? qs[hh][2 * lane + 1] : 0.f;
  }
  const double w2pi_l = lane < D / 2 ? w2pi[lane] : 0.0;
  __syncthreads();   // the query is in registers: the table may overwrite it
  // rotation table (w2pi is ready since the first barrier)
  for (int e = tid; e < 2 * (NPL / 2) * 32; e += NTH) {
    const int t = e % 32, hm = e / 32;                 // hm = half * (NPL / 2) + m2
    const int i0 = (hm / (NPL / 2)) * NPL + 2 * (hm % (NPL / 2));
    float4 v;
    double turns = static_cast<double>(t) * w2pi[i0];
    sincospif(2.0f * static_cast<float>(turns - floor(turns)), &v.y, &v.x);
    turns = static_cast<double>(t) * w2pi[i0 + 1];
    sincospif(2.0f * static_cast<float>(turns - floor(turns)), &v.w, &v.z);
    rtab[e] = v;
  }
  __syncthreads();   // table ready; omega read by all (wave 0's weight buffer is free)

  // ---- online softmax state --------------------------------------------------
  // mh[hh]: running max of head hh (wave-uniform). lane_l / lane_z: sums of p
  // and p z over this lane's tokens for head hd (lanes < 32; the upper half
  // holds copies). acc: the value product, rows 0..3 high parts of heads
  // 0..3, rows 4..7 remainders (as in kivi_mfma_kernel).
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mh[HG];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) mh[hh] = -INFINITY;
  float lane_l = 0.f, lane_z = 0.f;

  // qpage[wave][hh] = R(omega (T-1-t0)) q[hh]; lane < D/2 keeps its pair of
  // every head in qrot. rotate_q sets it from the angle; advance_q moves it to
  // the wave's next page (NW pages = NW * 32 tokens on) by the fixed rotation
  // R(-omega NW 32) of this lane's pair (dcs, dsn).
  float qrot[HG][2];
  float dcs = 1.f, dsn = 0.f;
  if (lane < D / 2) {
    const double turns = static_cast<double>(NW * kPage) * w2pi_l;
    sincospif(2.0f * static_cast<float>(turns - floor(turns)), &dsn, &dcs);
  }
  auto write_qpage = [&]() {
    if (lane < D / 2) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
        *reinterpret_cast<float2*>(&qpage[wave][2 * hh + (2 * lane) / HALF][(2 * lane) % HALF]) =
            float2{qrot[hh][0], qrot[hh][1]};
    }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
  };
  auto rotate_q = [&](int64_t t0) {
    if (lane < D / 2) {
      const double turns = static_cast<double>(Tb - 1 - t0) * w2pi_l;
      float sn, cs;
      sincospif(2.0f * static_cast<float>(turns - floor(turns)), &sn, &cs);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float q0 = qpair[hh][0], q1 = qpair[hh][1];
        qrot[hh][0] = fmaf(q0, cs, -(q1 * sn));
        qrot[hh][1] = fmaf(q0, sn, q1 * cs);
      }
    }
    write_qpage();
  };
  auto advance_q = [&]() {
    if (lane < D / 2) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float x = qrot[hh][0], y = qrot[hh][1];
        qrot[hh][0] = fmaf(x, dcs, y * dsn);
        qrot[hh][1] = fmaf(y, dcs, -(x * dsn));
      }
    }
    write_qpage();
  };

  // y: channels [part * CH, part * CH + CH) of this lane's half of its token
  // (dequantised); rotates them by the token's position (table), then adds
  // their key product against qpage into the four chains c
  const float* qrow = &qpage[wave][2 * hd + hf][0];
  auto rotate_mfma = [&](float* y, int part, floatx4* c) {
#pragma unroll
    for (int m2 = 0; m2 < CH / 4; ++m2) {
      const float4 r = rtab[(hf * (NPL / 2) + part * (CH / 4) + m2) * 32 + tk];
      const float x0 = y[4 * m2], x1 = y[4 * m2 + 1], x2 = y[4 * m2 + 2], x3 = y[4 * m2 + 3];
      y[4 * m2] = fmaf(x0, r.x, -(x1 * r.y));
      y[4 * m2 + 1] = fmaf(x0, r.y, x1 * r.x);
      y[4 * m2 + 2] = fmaf(x2, r.z, -(x3 * r.w));
      y[4 * m2 + 3] = fmaf(x2, r.w, x3 * r.z);
    }
    const float* qb = qrow + part * CH;
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) {
      const float4 bq = *reinterpret_cast<const float4*>(qb + 4 * i);
      c[0] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[4 * i], bq.x, c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[4 * i + 1], bq.y, c[1], 0, 0, 0);
      c[2] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[4 * i + 2], bq.z, c[2], 0, 0, 0);
      c[3] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[4 * i + 3], bq.w, c[3], 0, 0, 0);
    }
  };
  // the 4 scores of tokens 4((l/4)%8) + r for head hd (both halves added)
  auto finish_scores = [&](const floatx4* c) -> floatx4 {
    floatx4 s;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = (c[0][r] + c[1][r]) + (c[2][r] + c[3][r]);
      s[r] = v + xor32(v);
    }
    return s;
  };
  // folds 4 scores per lane (tokens 4((l/4)%8) + r, head hd; -inf = absent)
  // into the softmax state; returns the weights 2^(s - m)
  auto softmax = [&](floatx4 s) -> floatx4 {
    float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    float mine = mh[0];
#pragma unroll
    for (int hh = 1; hh < HG; ++hh) mine = hd == hh ? mh[hh] : mine;
    // the reference max of a head moves only when one of its scores exceeds
    // it by more than kMaxSlack (weights stay below 2^kMaxSlack; any
    // reference gives the same softmax); each lane's own maximum decides, the
    // maxima over the lanes of a head are formed only then
    if (__builtin_amdgcn_ballot_w64(pm > mine + kMaxSlack) != 0) {   // wave-uniform, rare
      // max over the 8 token quads of this half: lanes l ^ 4, l ^ 8, l ^ 16
      pm = fmaxf(pm, dpp<0x124>(pm));   // row_ror:4
      pm = fmaxf(pm, dpp<0x128>(pm));   // row_ror:8
      pm = fmaxf(pm, xor16(pm));
      const float m_new = fmaxf(mine, pm);
      float a_h[HG];
      bool grow = false;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float mn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_new), hh));
        grow |= mn > mh[hh];
        a_h[hh] = mn;
      }
      if (grow) {   // wave-uniform
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          const float a = fast_exp2(mh[hh] - a_h[hh]);
          mh[hh] = a_h[hh];
          a_h[hh] = a;
        }
        float a_mine = a_h[0];
#pragma unroll
        for (int hh = 1; hh < HG; ++hh) a_mine = hd == hh ? a_h[hh] : a_mine;
        lane_l *= a_mine;
        lane_z *= a_mine;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= a_h[r];   // rows 4g + r: head r
        }
      }
    }
    float mcur = mh[0];
#pragma unroll
    for (int hh = 1; hh < HG; ++hh) mcur = hd == hh ? mh[hh] : mcur;
    floatx4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = fast_exp2(s[r] - mcur);
    return w;
  };

  // P' (4 per lane, lanes < 32) -> LDS in the value operand's k order -> A
  // operand: rows 0..3 high part of head j, rows 4..7 remainder of head j-4
  auto weights_to_a = [&](floatx4 pw, bool permuted) -> bf16x8 {
    if (lane < 32) {
      uint32_t ph[2], pl[2];
      if (permuted) {   // element order {0,2,1,3} of each token quad (the fp4 converts' order)
        split_bf16(pw[0], pw[2], ph[0], pl[0]);
        split_bf16(pw[1], pw[3], ph[1], pl[1]);
      } else {
        split_bf16(pw[0], pw[1], ph[0], pl[0]);
        split_bf16(pw[2], pw[3], ph[1], pl[1]);
      }
      const int t0 = 4 * ((lane >> 2) & 7);
      *reinterpret_cast<uint2*>(&pbuf[wave][0][hd][t0]) = uint2{ph[0], ph[1]};
      *reinterpret_cast<uint2*>(&pbuf[wave][1][hd][t0]) = uint2{pl[0], pl[1]};
    }
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    uint4 v = uint4{0u, 0u, 0u, 0u};
    if (j < 8) v = *reinterpret_cast<const uint4*>(&pbuf[wave][j >> 2][j & 3][8 * g]);
    return __builtin_bit_cast(bf16x8, v);
  };

  // page k of this wave starts at token t0; its qpage is set exactly every 16th
  // page and advanced by one fixed rotation in between (the fp32 drift over 15
  // steps stays near the rounding of one rotation)
  auto process_page = [&](const uint8_t* pg, int64_t t0, int k) {
    if ((k & 15) == 0) rotate_q(t0);
    else advance_q();
    floatx4 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    const float* sp = reinterpret_cast<const float*>(pg + PG::OFF_KS) + hf * HALF;
    const float* zp = reinterpret_cast<const float*>(pg + PG::OFF_KZ) + hf * HALF;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      // this lane's token row, channels [part * CH, +CH) of its half: CH / 16 words
      float y[CH];
#pragma unroll
      for (int w = 0; w < CH / 16; ++w) {
        const int cw = part * CH + 16 * w;   // first channel of the word within the half
        const uint32_t word = *reinterpret_cast<const uint32_t*>(pg + krow_off<CPR_K>(tk, hf * (D / 8) + cw / 4));
        // nibble n of ev / od: the code of channel 2n / 2n + 1 of the word, so
        // byte q4 of ev holds channels 4 q4 and 4 q4 + 2, of od 4 q4 + 1 and 4 q4 + 3
        const uint32_t ev = word & 0x33333333u, od = (word >> 2) & 0x33333333u;
        const float2 ce[4] = {codes2_f32<0>(ev), codes2_f32<1>(ev), codes2_f32<2>(ev), codes2_f32<3>(ev)};
        const float2 co[4] = {codes2_f32<0>(od), codes2_f32<1>(od), codes2_f32<2>(od), codes2_f32<3>(od)};
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 sv = *reinterpret_cast<const float4*>(sp + cw + 4 * q4);
          const float4 zv = *reinterpret_cast<const float4*>(zp + cw + 4 * q4);
          y[16 * w + 4 * q4 + 0] = fmaf(ce[q4].x, sv.x, zv.x);
          y[16 * w + 4 * q4 + 1] = fmaf(co[q4].x, sv.y, zv.y);
          y[16 * w + 4 * q4 + 2] = fmaf(ce[q4].y, sv.z, zv.z);
          y[16 * w + 4 * q4 + 3] = fmaf(co[q4].y, sv.w, zv.w);
        }
      }
      rotate_mfma(y, part, c);
    }
    floatx4 sc = finish_scores(c);
    if (in_page && Tb - t0 < kPage) {   // the query's own token is in this page
      const int nvalid = static_cast<int>(Tb - t0);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * ((lane >> 2) & 7) + r >= nvalid) sc[r] = -INFINITY;
    }
    const floatx4 w = softmax(sc);
    // P' = p * s_t; sums of p and p * z_t (lanes < 32 own the tokens)
    const int t0q = 4 * ((lane >> 2) & 7);
    const float4 vs = *reinterpret_cast<const float4*>(pg + PG::OFF_VS + 4 * t0q);
    const float4 vz = *reinterpret_cast<const float4*>(pg + PG::OFF_VZ + 4 * t0q);
    if (lane < 32) {
      lane_l += (w[0] + w[1]) + (w[2] + w[3]);
      lane_z = fmaf(w[0], vz.x, fmaf(w[1], vz.y, fmaf(w[2], vz.z, fmaf(w[3], vz.w, lane_z))));
    }
    const floatx4 pv = {w[0] * vs.x, w[1] * vs.y, w[2] * vs.z, w[3] * vs.w};
    const bf16x8 ap = weights_to_a(pv, true);
    // value codes of tokens {8g..8g+7} of channel 16 nt + j (bytes 2g, 2g+1)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t x = *reinterpret_cast<const uint16_t*>(pg + PG::OFF_VC + (16 * nt + j) * VROW + 2 * g);
      const uint32_t y0 = x & 0x3333u, y1 = (x >> 2) & 0x3333u;
      const uint4 bw = uint4{bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 0)),
                             bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 0)),
                             bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y0, 2.0f, 1)),
                             bits32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(y1, 2.0f, 1))};
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
    }
  };

  // residual step: tokens 0..7 of the step are lanes with tk < 8
  auto process_step = [&](int hs) {
    const int64_t t0 = q_tokens + static_cast<int64_t>(hs) * RSTEP;
    const int nv = static_cast<int>(Tb - t0 < RSTEP ? Tb - t0 : RSTEP);
    rotate_q(t0);
    floatx4 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(wring + (tk & 7) * 2 * D) + hf * HALF;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      float y[CH];
#pragma unroll
      for (int i = 0; i < CH / 8; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + part * CH + 8 * i);
        unpack_bf16x8(v, y + 8 * i);
      }
      rotate_mfma(y, part, c);
    }
    floatx4 s = finish_scores(c);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = 4 * ((lane >> 2) & 7) + r < nv ? s[r] : -INFINITY;
    const floatx4 w = softmax(s);
    if (lane < 32) lane_l += (w[0] + w[1]) + (w[2] + w[3]);   // absent tokens: 0
    const bf16x8 ap = weights_to_a(w, false);
    // value rows: tokens 8g..8g+7 exist for g = 0 only (absent rows are zero)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint4 bw = uint4{0u, 0u, 0u, 0u};
      if (g == 0) {
        const uint16_t* vr = reinterpret_cast<const uint16_t*>(wring + RSTEP * 2 * D) + 16 * nt + j;
        bw = uint4{uint32_t(vr[0]) | (uint32_t(vr[D]) << 16), uint32_t(vr[2 * D]) | (uint32_t(vr[3 * D]) << 16),
                   uint32_t(vr[4 * D]) | (uint32_t(vr[5 * D]) << 16), uint32_t(vr[6 * D]) | (uint32_t(vr[7 * D]) << 16)};
      }
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, __builtin_bit_cast(bf16x8, bw), acc[nt], 0, 0, 0);
    }
  };

  // ---- residual steps first (all of this wave's, in the page buffers), then
  // the pages; a wave with steps requests its first page after them ------------
  for (int hs = my_wave; hs < n_steps; hs += waves_total) {
    if (hs != my_wave) {
      wait_lds();
      __builtin_amdgcn_wave_barrier();
      issue_step(hs);
    }
    wait_vm<0>();
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    process_step(hs);
  }
  if (has_step && n_mine > 0) {
    wait_lds();   // the step rows have been read
    __builtin_amdgcn_wave_barrier();
    issue_page(0);
  }
#pragma unroll 1
  for (int k = 0; k < n_mine; ++k) {
    wait_lds();
    __builtin_amdgcn_wave_barrier();
    const bool next = k + 1 < n_mine;
    if (next) issue_page(k + 1);
    if (next) wait_vm<PG::DMA>();
    else wait_vm<0>();
    __builtin_amdgcn_wave_barrier();
    process_page(wbuf + (k % 2) * PG::BYTES, static_cast<int64_t>(pg0 + wave + NW * k) * kPage, k);
  }
  wait_lds();

  // ---- wave epilogue: per-head sums (lanes < 32 with head hd) ----------------
  float lsum[HG], zsum[HG];
  {
    float l_ = lane < 32 ? lane_l : 0.f, z_ = lane < 32 ? lane_z : 0.f;
    // sum over the 8 token quads: lanes l ^ 4, l ^ 8, l ^ 16, then l ^ 32
    l_ += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, l_), (0x04 << 10) | 0x1F));
    z_ += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, z_), (0x04 << 10) | 0x1F));
    l_ += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, l_), (0x08 << 10) | 0x1F));
    z_ += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, z_), (0x08 << 10) | 0x1F));
    l_ += xor16(l_);
    z_ += xor16(z_);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      lsum[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_), hh));
      zsum[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z_), hh));
    }
  }
  finish_unit<D, HG, NW>(p, acc, mh, lsum, zsum, arena, last_block, b, qi, h, split);
}


// rows: grid rows (batch * queries / qn); qn: queries per block (2: GQA 4,
// keys without rotation; 4: kivi_deq_kernel, 2-bit values, d <= 128)
template <int KB, int VB, int D, bool ROPE>
hipError_t by_hg(const MfmaParams& p, int hg, int rows, int qn, hipStream_t st) {
  dim3 grid(p.splits, p.kv_heads, rows);
  switch (hg) {
    case 1: hipLaunchKernelGGL((kivi_mfma_kernel<KB, VB, D, 1, ROPE>), grid, dim3(64 * kivi_waves(KB, VB, D, 1, ROPE)), 0, st, p); break;
    case 2: hipLaunchKernelGGL((kivi_mfma_kernel<KB, VB, D, 2, ROPE>), grid, dim3(64 * kivi_waves(KB, VB, D, 2, ROPE)), 0, st, p); break;
    case 4:
      if constexpr (!ROPE && D <= 128) {
        if (qn == 4) {   // four queries per block over dequantised keys
          hipLaunchKernelGGL((kivi_deq_kernel<KB, VB, D>), grid, dim3(512), 0, st, p);
          break;
        }
      }
      if constexpr (!ROPE) {
        if (qn == 2) {
          hipLaunchKernelGGL((kivi_mfma_kernel<KB, VB, D, 4, ROPE, 2>), grid, dim3(64 * kivi_waves(KB, VB, D, 4, ROPE)), 0, st, p);
          break;
        }
      }
      hipLaunchKernelGGL((kivi_mfma_kernel<KB, VB, D, 4, ROPE>), grid, dim3(64 * kivi_waves(KB, VB, D, 4, ROPE)), 0, st, p);
      break;
    default: hipLaunchKernelGGL((kivi_mfma_kernel<KB, VB, D, 8, ROPE>), grid, dim3(64 * kivi_waves(KB, VB, D, 8, ROPE)), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t by_d(const MfmaParams& p, int d, int hg, int rows, int qn, hipStream_t st) {
  switch (d) {
    case 64: return by_hg<KB, VB, 64, false>(p, hg, rows, qn, st);
    case 128: return by_hg<KB, VB, 128, false>(p, hg, rows, qn, st);
    default: return by_hg<KB, VB, 256, false>(p, hg, rows, qn, st);
  }
}

hipError_t by_d_rope(const MfmaParams& p, int d, int hg, int batch, hipStream_t st) {
  if (hg == 4) {   // dense-score kernel
    dim3 grid(p.splits, p.kv_heads, batch);
    if (d == 64) hipLaunchKernelGGL((rope4_kernel<64, kRopeWaves>), grid, dim3(64 * kRopeWaves), 0, st, p);
    else hipLaunchKernelGGL((rope4_kernel<128, kRopeWaves>), grid, dim3(64 * kRopeWaves), 0, st, p);
    return hipGetLastError();
  }
  return d == 64 ? by_hg<2, 2, 64, true>(p, hg, batch, 1, st) : by_hg<2, 2, 128, true>(p, hg, batch, 1, st);
}

}  // namespace

bool mfma_path(const Geometry& g) {
  if (g.scheme != KVQ_KIVI || g.d < 64 || g.in_bytes != 2) return false;
  if (g.outliers) return false;   // dense-and-sparse pages: the generic kernel
  if (g.vbits != 2 && g.vbits != 4) return false;          // 3-bit values: the generic kernel
  if (g.rope == 0.0) return g.bits == 2 || g.bits == 4;   // value bits: 2 or 4, <= key bits
  return g.bits == 2 && g.d <= 128;   // rotary keys: 2-bit pages, head_dim 64 or 128
}

MfmaPlan mfma_plan(const Geometry& g, int64_t tokens, int32_t requested) {
  MfmaPlan pl{};
  const int64_t q = kivi_quantised(tokens, g.residual);
  pl.pages = static_cast<int32_t>(q / kPage);
  pl.chunks = static_cast<int32_t>((tokens - q + 7) / 8);     // residual 8-token steps
  int64_t s;
  if (requested > 0) {
    s = requested;
  } else {
    // about one resident round of blocks (256 CUs), >= 8 pages each
    const int64_t units = static_cast<int64_t>(g.batch) * g.kv_heads;
    const bool rope = g.rope != 0.0;
    // rotary keys at GQA 4 run rope4_kernel (three blocks per CU)
    // (2-bit pages without rotation run eight-wave blocks: one per CU for short
    // caches, where fewer blocks mean fewer set-ups and partials to merge --
    // 19.8 vs 20.6 us at batch 16, 124 pages per (sequence, KV head) -- and two
    // per CU from 192 pages on, where more waves keep the SIMDs busier: 31.2
    // vs 32.9 us at 252 pages, 98.5 vs 117.7 us at 1020 pages)
    const int64_t per_cu = rope && g.hg == 4 ? 3
                         : kivi_waves(g.bits, g.vbits, g.d, g.hg, rope) == 8 ? (pl.pages >= 192 ? 2 : 1)
                         : kivi_blocks_per_cu(g.bits, g.d, rope);
    const int64_t target = 256 * per_cu;
    s = (target + units - 1) / units;
    const int64_t cap = (pl.pages + 7) / 8;
    if (s > cap) s = cap;
  }
  if (s > pl.pages) s = pl.pages;
  pl.page_splits = static_cast<int32_t>(s < 1 ? 1 : s);
  pl.ring_splits = 0;
  pl.ring_splits_max = 0;
  return pl;
}

bool mfma_fused_append_ok(const Geometry& g) {
  return mfma_path(g) && !(g.rope != 0.0 && g.hg == 4);   // not rope4_kernel
}

bool mfma_multi_ok(const Geometry& g, int64_t tokens, int32_t nq) {
  return mfma_path(g) && nq >= 1 && nq <= tokens;
}

hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const int32_t nq = a.nq > 1 ? a.nq : 1;
  // several queries per sequence: batch * nq rows share the chip, so the
  // split count is planned for that many rows (never more splits than the
  // one-query plan, whose workspace nq copies of hold the partials)
  // two queries per block: GQA 4, keys without rotation, an even number of
  // queries (their tokens in the ring or in pages)
  // four per block over dequantised keys (kivi_deq_kernel): a multiple of
  // four queries of a uniform batch, 2-bit values, head_dim <= 128 (at the
  // kivi2 shape 4 queries 33.9 us against 35.5 with two per block, 8: 44.0
  // against 69.0, 16: 84.5 against 136.1)
  const bool pairs = nq >= 2 && nq % 2 == 0 && g.hg == 4 && a.rope_theta == 0.0;
  const bool fours = pairs && nq % 4 == 0 && g.d <= 128 && !a.seq_tokens;
  const int qn = fours ? 4 : pairs ? 2 : 1;
  Geometry rows = g;
  rows.batch = g.batch * nq / qn;
  const MfmaPlan pl = mfma_plan(rows, a.tokens, a.requested_splits);
  MfmaParams p{};
  p.pm = a.pm;
  p.layer_base = a.layer_base;
  p.q = static_cast<const uint8_t*>(a.q);
  p.out = a.out;
  p.partials = reinterpret_cast<float*>(a.workspace + workspace_partials_offset(g));
  p.counters = reinterpret_cast<int*>(a.workspace);
  p.slab_bytes = g.slab_bytes;
  p.page_bytes = g.page_bytes;
  p.ring_base = g.pages_per_slab * g.page_bytes;
  p.ring_slots = g.ring_slots;
  p.T = a.tokens;
  p.seq_tokens = a.seq_tokens;
  p.q_tokens = static_cast<int64_t>(pl.pages) * kPage;
  p.n_pages = pl.pages;
  p.n_steps = pl.chunks;
  p.residual = g.residual;
  p.nq = nq;
  p.splits = pl.page_splits;
  p.kv_heads = g.kv_heads;
  p.q_heads = g.q_heads;
  p.q_bf16 = a.q_dtype == KVQ_BF16;
  p.qscale = a.sm_scale * kLog2e;
  p.rope_theta = a.rope_theta;
  p.new_tok = -1;
  if (a.k_new) {   // fused one-token append (uniform batch, one query)
    p.k_new = static_cast<const uint8_t*>(a.k_new);
    p.v_new = static_cast<const uint8_t*>(a.v_new);
    p.new_tok = a.tokens - 1;
  }
  const int grid_rows = g.batch * nq / qn;
  // long chunks (a multiple of 32 queries whose rows of 32 fill the chip):
  // one block per (sequence, KV head, 32 queries), one split
  if (fours && g.vbits == 2 && g.d == 128 && nq % 32 == 0 &&
      static_cast<int64_t>(g.batch) * (nq / 32) * g.kv_heads >= 256) {
    p.splits = 1;
    const dim3 grid(1, g.kv_heads, g.batch * (nq / 32));
    if (g.bits == 2) hipLaunchKernelGGL((kivi_chunk_kernel<2>), grid, dim3(512), 0, st, p);
    else hipLaunchKernelGGL((kivi_chunk_kernel<4>), grid, dim3(512), 0, st, p);
    return hipGetLastError();
  }
  if (a.rope_theta > 0.0) return by_d_rope(p, g.d, g.hg, grid_rows, st);
  if (g.bits == 2) return by_d<2, 2>(p, g.d, g.hg, grid_rows, qn, st);
  return g.vbits == 2 ? by_d<4, 2>(p, g.d, g.hg, grid_rows, qn, st)
                      : by_d<4, 4>(p, g.d, g.hg, grid_rows, qn, st);
}

}  // namespace kvq
