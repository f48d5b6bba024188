// Decode attention over KIVI 2/4-bit pages on the matrix cores (gfx950).
//
// Same result as the generic kernel (softmax(sm_scale q.K^) . V^ over the
// dequantised cache, "Quantizing the KV cache", going deeper), organised for
// v_mfma_f32_16x16x32_f16. For one 32-token page of one (sequence, KV head):
//
//   keys:   S^T[t][h] = sum_c code_tc * q'_hc + b_h,  q'_hc = q_hc s_c,
//           b_h = sum_c q_hc z_c          (per-channel scale/offset folded in)
//           A = key codes [16 tokens x 32 channels] (exact small integers in
//           f16), B = q'^T [32 channels x 16 columns]: columns 0..HG-1 hold the
//           f16 "hi" part of q' of each GQA head, columns HG..2HG-1 the f16 "lo"
//           remainder (q' - hi), so hi + lo carries ~22 bits; the two column
//           groups are added after the product.
//   values: O[h][c] += sum_t P'[h][t] code_tc,  P'_ht = p_ht s_t, plus
//           sum_t p_ht z_t added to every channel at the end.
//           A = P' [16 rows x 32 tokens] (rows 0..HG-1 hi, HG..2HG-1 lo),
//           B = value codes [32 tokens x 16 channels].
//
// Operand layouts of v_mfma_f32_16x16x32_f16 (wave64): lane l holds
// A[l%16][8(l/16)+i], B[8(l/16)+i][l%16] (i = 0..7) and C[4(l/16)+r][l%16]
// (r = 0..3). Computing S^T (tokens as rows) leaves lane (j, g) = (l%16, l/16)
// holding the scores of head j for tokens {4g..4g+3} and {16+4g..16+4g+3}: the
// same lane and token set the P.V A-operand needs, so P never moves between
// lanes. Value codes are fed in that token order: for channel c, tokens
// 4g..4g+3 are byte g of the channel's 2-bit run (bytes 2g, 2g+1 at 4 bits).
//
// Codes become exact f16 integers with the scaled converts: a 2-bit code in
// the low bits of an FP4 E2M1 nibble is code/2 (scale 2), a 4-bit code in an
// FP8 E4M3 byte is code * 2^-9 (scale 512). Both convert two fields per
// instruction; the resulting channel order within 8 is {0,2,1,3,4,6,5,7}, and
// q' is laid out in the same order.
//
// Online softmax per head (log2 domain: q pre-scaled by sm_scale*log2 e). The
// output accumulators are only rescaled when some head's running max grows.
//
// The residual ring (unquantised, input dtype) is handled by dedicated blocks
// on the vector ALUs; every block writes a partial (m, l, o) and a merge
// kernel combines them, or the single block writes the output directly.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct MfmaParams {
  const uint8_t* layer_base;
  const uint8_t* q;
  float* out;
  float* partials;
  int64_t slab_bytes, page_bytes, ring_base, ring_slots;
  int64_t T, q_tokens;
  int32_t n_pages, n_chunks;      // quantised pages, ring chunks of 32 tokens
  int32_t page_splits, splits;    // blocks [0, page_splits) take pages, the rest ring chunks
  int32_t kv_heads, q_heads;
  int32_t off_ks, off_kz, off_vc, off_vs, off_vz;
  int32_t q_bf16, in_bf16;
  float qscale;
};

// Orders LDS traffic of one wave: the writes above are visible to the reads
// below (LDS executes a wave's instructions in order; this stops the compiler
// from moving memory operations across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ half8 cat4(half2v a, half2v b, half2v c, half2v d) {
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 16 two-bit codes (one word) -> two 8-channel fragments, channel order
// {0,2,1,3,4,6,5,7} within each 8.
__device__ __forceinline__ void codes2_frags(uint32_t w, half8& f0, half8& f1) {
  const uint32_t y0 = w & 0x33333333u, y1 = (w >> 2) & 0x33333333u;
  f0 = cat4(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 0),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 0),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 1),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 1));
  f1 = cat4(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 2),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 2),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 3),
            __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 3));
}

// 8 four-bit codes (one word) -> one fragment, channel order {0,2,1,3,4,6,5,7}.
__device__ __forceinline__ half8 codes4_frag(uint32_t w) {
  const uint32_t y0 = w & 0x0F0F0F0Fu, y1 = (w >> 4) & 0x0F0F0F0Fu;
  return cat4(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y0, 512.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y1, 512.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y0, 512.0f, true),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y1, 512.0f, true));
}

// Sum over the 16 lanes of each DPP row (all lanes receive it).
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Value of lane l ^ 32.
__device__ __forceinline__ float xor32(float v) {
  const int lane = threadIdx.x & 63;
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                            false, false);
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// Value of lane l ^ 16 (within each half of the wave).
__device__ __forceinline__ float xor16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                               (0x10 << 10) | 0x1F));
}

template <int SHIFT>
__device__ __forceinline__ float row_shl(float v) {  // lane l gets lane l+SHIFT of its row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x100 + SHIFT, 0xF, 0xF, false));
}

template <int SHIFT>
__device__ __forceinline__ uint32_t row_shr_u(uint32_t v) {  // lane l gets lane l-SHIFT of its row
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x110 + SHIFT,
                                                           0xF, 0xF, false));
}

// f32 pair -> packed f16 (hi) and packed f16 remainder (lo) with hi + lo ~ x.
__device__ __forceinline__ void split_hilo(float a, float b, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a, b);
  const auto r = __builtin_amdgcn_cvt_pkrtz(a - static_cast<float>(h[0]), b - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float load_in(const uint8_t* base, int64_t idx, int bf16) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

template <int BITS, int D, int HG>
__global__ __launch_bounds__(kThreads) void kivi_mfma_kernel(MfmaParams p) {
  static_assert(BITS == 2 || BITS == 4, "2- or 4-bit pages");
  static_assert(2 * HG <= 16, "hi and lo columns of the GQA group fit one tile");
  constexpr int KS = D / 32;             // k-steps of the key product
  constexpr int NT = D / 16;             // channel tiles of the value product
  constexpr int CPG = D / 4;             // key channels per lane group
  constexpr int KROW = D * BITS / 8;     // bytes per key token row
  constexpr int KW = CPG * BITS / 32;    // key-code words per lane per 16-token tile
  constexpr int VROW = 32 * BITS / 8;    // bytes per value channel column
  constexpr int COMBOS = HG * 4 * KS;    // (head, lane group, k-step) fold units
  constexpr int REPS = (COMBOS + 63) / 64;
  static_assert(KW >= 1, "at least one word per lane");

  __shared__ __attribute__((aligned(16))) float qs[HG][D];
  __shared__ __attribute__((aligned(16))) uint32_t frag[kWaves][KS][64][4];  // B fragments of q'
  __shared__ float wp[kWaves][HG][32];                                      // ring: p per token
  __shared__ float red[kWaves][HG][D + 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const uint8_t* slab = p.layer_base + (static_cast<int64_t>(b) * p.kv_heads + h) * p.slab_bytes;

  for (int i = tid; i < HG * D; i += kThreads) {
    const int gg = i / D, c = i % D;
    const int64_t qi = (static_cast<int64_t>(b) * p.q_heads + h * HG + gg) * D + c;
    qs[gg][c] = load_in(p.q, qi, p.q_bf16) * p.qscale;
  }
  // zero B-fragment columns >= 2*HG once; they are never written again
  for (int i = lane; i < KS * 64; i += 64) {
    const int ks = i / 64, ln = i % 64;
    if ((ln & 15) >= 2 * HG) {
      frag[wave][ks][ln][0] = frag[wave][ks][ln][1] = 0u;
      frag[wave][ks][ln][2] = frag[wave][ks][ln][3] = 0u;
    }
  }
  __syncthreads();

  float m[HG], lsum[HG], zsum[HG];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = -INFINITY;
    lsum[hh] = 0.f;
    zsum[hh] = 0.f;
  }
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (split < p.page_splits) {
    // ---------------- quantised pages on the matrix cores -------------------
    // fold units handled by this lane: (head, lane group, k-step) -> 8 channels
    float qreg[REPS][8];
#pragma unroll
    for (int r = 0; r < REPS; ++r) {
      const int cidx = lane + 64 * r;
      const int fh = cidx / (4 * KS), fg = (cidx / KS) % 4, fk = cidx % KS;
      const int c0 = fg * CPG + 8 * fk;
#pragma unroll
      for (int i = 0; i < 8; ++i) qreg[r][i] = cidx < COMBOS ? qs[fh][c0 + i] : 0.f;
    }
    const int pg0 = static_cast<int>(static_cast<int64_t>(split) * p.n_pages / p.page_splits);
    const int pg1 = static_cast<int>(static_cast<int64_t>(split + 1) * p.n_pages / p.page_splits);

#pragma unroll 1
    for (int pi = pg0 + wave; pi < pg1; pi += kWaves) {
      const uint8_t* pg = slab + static_cast<int64_t>(pi) * p.page_bytes;
      // ---- loads ----
      uint32_t kc[2][KW];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(pg + (16 * mt + j) * KROW + g * (KW * 4));
#pragma unroll
        for (int w = 0; w < KW; ++w) kc[mt][w] = src[w];
      }
      float ksv[REPS][8], kzv[REPS][8];
#pragma unroll
      for (int r = 0; r < REPS; ++r) {
        const int cidx = lane + 64 * r;
        const int fg = (cidx / KS) % 4, fk = cidx % KS;
        const int c0 = fg * CPG + 8 * fk;
        const float4* sp = reinterpret_cast<const float4*>(pg + p.off_ks) + c0 / 4;
        const float4* zp = reinterpret_cast<const float4*>(pg + p.off_kz) + c0 / 4;
        const float4 s0 = sp[0], s1 = sp[1], z0 = zp[0], z1 = zp[1];
        ksv[r][0] = s0.x; ksv[r][1] = s0.y; ksv[r][2] = s0.z; ksv[r][3] = s0.w;
        ksv[r][4] = s1.x; ksv[r][5] = s1.y; ksv[r][6] = s1.z; ksv[r][7] = s1.w;
        kzv[r][0] = z0.x; kzv[r][1] = z0.y; kzv[r][2] = z0.z; kzv[r][3] = z0.w;
        kzv[r][4] = z1.x; kzv[r][5] = z1.y; kzv[r][6] = z1.z; kzv[r][7] = z1.w;
      }
      // value codes: channel NT*j + nt, the words holding tokens {4g..} and {16+4g..}
      uint32_t vlo[NT], vhi[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t* col = reinterpret_cast<const uint32_t*>(pg + p.off_vc + (NT * j + nt) * VROW);
        if constexpr (BITS == 2) {
          vlo[nt] = col[0];
          vhi[nt] = col[1];
        } else {
          vlo[nt] = col[g >> 1];
          vhi[nt] = col[2 + (g >> 1)];
        }
      }
      const float4* vsp = reinterpret_cast<const float4*>(pg + p.off_vs);
      const float4* vzp = reinterpret_cast<const float4*>(pg + p.off_vz);
      const float4 vs0 = vsp[g], vs1 = vsp[4 + g], vz0 = vzp[g], vz1 = vzp[4 + g];

      // ---- q' = q * s per channel, split hi/lo into B fragments; bias q.z ----
      float bias_part[REPS];
#pragma unroll
      for (int r = 0; r < REPS; ++r) {
        const int cidx = lane + 64 * r;
        const int fh = cidx / (4 * KS), fg = (cidx / KS) % 4, fk = cidx % KS;
        float qp[8];
        float bp = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          qp[i] = qreg[r][i] * ksv[r][i];
          bp = fmaf(qreg[r][i], kzv[r][i], bp);
        }
        bias_part[r] = bp;
        // fragment order {0,2,1,3,4,6,5,7}
        uint32_t hi[4], lo[4];
        split_hilo(qp[0], qp[2], hi[0], lo[0]);
        split_hilo(qp[1], qp[3], hi[1], lo[1]);
        split_hilo(qp[4], qp[6], hi[2], lo[2]);
        split_hilo(qp[5], qp[7], hi[3], lo[3]);
        if (cidx < COMBOS) {
          uint32_t* dh = frag[wave][fk][16 * fg + fh];
          uint32_t* dl = frag[wave][fk][16 * fg + HG + fh];
          *reinterpret_cast<uint4*>(dh) = uint4{hi[0], hi[1], hi[2], hi[3]};
          *reinterpret_cast<uint4*>(dl) = uint4{lo[0], lo[1], lo[2], lo[3]};
        }
      }
      // bias per head: the fold units of head fh are contiguous lanes
      float bias_h[HG];
      {
        constexpr int PER_HEAD = 4 * KS;   // lanes (units) per head
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) bias_h[hh] = 0.f;
#pragma unroll
        for (int r = 0; r < REPS; ++r) {
          float v = bias_part[r];
          if constexpr (PER_HEAD == 8) {
            v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
          } else {
            v = row_sum16(v);
            if constexpr (PER_HEAD == 32) v += xor16(v);
          }
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            const int first = hh * PER_HEAD - 64 * r;   // first lane of head hh in this rep
            if (first >= 0 && first < 64)
              bias_h[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), first));
          }
        }
      }
      wave_lds_sync();
      half8 bq[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const half8*>(frag[wave][ks][lane]);

      // ---- scores S^T = codes x q'^T ----
      floatx4 sc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        floatx4 c = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BITS == 2) {
#pragma unroll
          for (int w = 0; w < KW; ++w) {
            half8 a0, a1;
            codes2_frags(kc[mt][w], a0, a1);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bq[2 * w], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bq[2 * w + 1], c, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int w = 0; w < KW; ++w)
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes4_frag(kc[mt][w]), bq[w], c, 0, 0, 0);
        }
        sc[mt] = c;
      }
      // hi + lo columns, plus the bias of this lane's head
      float bias_j = 0.f;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) bias_j = j == hh ? bias_h[hh] : bias_j;
      float s[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[4 * mt + r] = sc[mt][r] + row_shl<HG>(sc[mt][r]) + bias_j;

      // ---- online softmax (lanes j < HG hold head j) ----
      float pmax = s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) pmax = fmaxf(pmax, s[i]);
      pmax = fmaxf(pmax, xor16(pmax));
      pmax = fmaxf(pmax, xor32(pmax));
      float m_new[HG];
      bool grow = false;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float pm = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pmax), hh));
        m_new[hh] = fmaxf(m[hh], pm);
        grow = grow || (m_new[hh] > m[hh]);
      }
      if (grow) {   // wave-uniform
        float alpha[HG];
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          alpha[hh] = exp2f(m[hh] - m_new[hh]);
          lsum[hh] *= alpha[hh];
          zsum[hh] *= alpha[hh];
          m[hh] = m_new[hh];
        }
        // accumulator rows 4g+r: head (4g+r) % HG (hi rows then lo rows)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a = 1.f;
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) a = ((4 * g + r) % HG == hh) ? alpha[hh] : a;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][r] *= a;
        }
      }
      float m_j = 0.f;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) m_j = j == hh ? m[hh] : m_j;
      const float vsv[8] = {vs0.x, vs0.y, vs0.z, vs0.w, vs1.x, vs1.y, vs1.z, vs1.w};
      const float vzv[8] = {vz0.x, vz0.y, vz0.z, vz0.w, vz1.x, vz1.y, vz1.z, vz1.w};
      float pv[8];
      float lpart = 0.f, zpart = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pe = exp2f(s[i] - m_j);
        lpart += pe;
        zpart = fmaf(pe, vzv[i], zpart);
        pv[i] = pe * vsv[i];
      }
      // per-head partial sums stay per lane (lanes j < HG); reduced at the end
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        lsum[hh] += j == hh ? lpart : 0.f;
        zsum[hh] += j == hh ? zpart : 0.f;
      }
      // P' into A fragments: token order {4g+0,4g+2,4g+1,4g+3, 16+4g+0,...}
      uint32_t ph[4], pl[4];
      split_hilo(pv[0], pv[2], ph[0], pl[0]);
      split_hilo(pv[1], pv[3], ph[1], pl[1]);
      split_hilo(pv[4], pv[6], ph[2], pl[2]);
      split_hilo(pv[5], pv[7], ph[3], pl[3]);
      uint32_t pa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo_from_head = row_shr_u<HG>(pl[i]);   // lane j gets lane j-HG
        pa[i] = j < HG ? ph[i] : (j < 2 * HG ? lo_from_head : 0u);
      }
      const half8 ap = __builtin_bit_cast(half8, uint4{pa[0], pa[1], pa[2], pa[3]});

      // ---- P' x value codes ----
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        half8 bv;
        if constexpr (BITS == 2) {
          // byte g of each word: tokens 4g..4g+3 and 16+4g..16+4g+3
          const uint32_t x = __builtin_amdgcn_perm(vhi[nt], vlo[nt], 0x0C0C0400u + 0x0101u * g);
          const uint32_t y0 = x & 0x3333u, y1 = (x >> 2) & 0x3333u;
          bv = cat4(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 0),
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 0),
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 1),
                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 1));
        } else {
          // bytes 2g,2g+1 (tokens 4g..4g+3) and 8+2g, 9+2g (tokens 16+4g..)
          const uint32_t sh = (g & 1) * 2;
          const uint32_t sel = (0x0100u + 0x0101u * sh) | ((0x0504u + 0x0101u * sh) << 16);
          const uint32_t x = __builtin_amdgcn_perm(vhi[nt], vlo[nt], sel);
          bv = codes4_frag(x);
        }
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, bv, acc[nt], 0, 0, 0);
      }
    }

    // ---- wave epilogue: rows (hi, lo) -> heads; per-lane sums -> per head ----
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float l_ = lsum[hh], z_ = zsum[hh];
      l_ += xor16(l_);
      l_ += xor32(l_);
      z_ += xor16(z_);
      z_ += xor32(z_);
      lsum[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_), hh));
      zsum[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, z_), hh));
    }
    // acc rows 4g+r: row < HG is head row (hi), HG <= row < 2HG is head row-HG (lo)
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
          x += xor16(x);          // rows 0-3 (g=0) + rows 4-7 (g=1)
        } else {
          x += xor32(x);          // rows 0-7 (g=0,1) + rows 8-15 (g=2,3)
        }
        v[r] = x;
      }
      const int c = NT * j + nt;
      if (4 * g < HG) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = 4 * g + r;
          float zz = 0.f;   // sum_t p z_t of head hh goes to every channel
#pragma unroll
          for (int k = 0; k < HG; ++k) zz = hh == k ? zsum[k] : zz;
          if (hh < HG) red[wave][hh][2 + c] = v[r] + zz;
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        red[wave][hh][0] = m[hh];
        red[wave][hh][1] = lsum[hh];
      }
    }
    __syncthreads();
  } else {
    // ---------------- residual ring on the vector ALUs ----------------------
    const int chunk0 = (split - p.page_splits);
    const int n_ring_blocks = p.splits - p.page_splits;
    const int tok = lane & 31, hf = lane >> 5;
    constexpr int HALF = D / 2;
    constexpr int CPL = D / 64;
    float o[HG][CPL];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[hh][c] = 0.f;
    const int ib = p.in_bf16 ? 2 : 4;
#pragma unroll 1
    for (int ch = chunk0 + n_ring_blocks * wave; ch < p.n_chunks; ch += n_ring_blocks * kWaves) {
      const int64_t t0 = p.q_tokens + static_cast<int64_t>(ch) * 32;
      const int nv = static_cast<int>(p.T - t0 < 32 ? p.T - t0 : 32);
      float sc[HG];
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) sc[hh] = 0.f;
      if (tok < nv) {
        const int64_t slot = (t0 + tok) % p.ring_slots;
        const uint8_t* row = slab + p.ring_base + slot * D * ib;
#pragma unroll 1
        for (int c = hf * HALF; c < hf * HALF + HALF; c += 8) {
          float x[8];
          if (p.in_bf16) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(row + c * 2), x);
          } else {
            const float4 a = *reinterpret_cast<const float4*>(row + c * 4);
            const float4 bq = *reinterpret_cast<const float4*>(row + c * 4 + 16);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = bq.x; x[5] = bq.y; x[6] = bq.z; x[7] = bq.w;
          }
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            const float4 q0 = *reinterpret_cast<const float4*>(&qs[hh][c]);
            const float4 q1 = *reinterpret_cast<const float4*>(&qs[hh][c + 4]);
            float a = sc[hh];
            a = fmaf(q0.x, x[0], a); a = fmaf(q0.y, x[1], a);
            a = fmaf(q0.z, x[2], a); a = fmaf(q0.w, x[3], a);
            a = fmaf(q1.x, x[4], a); a = fmaf(q1.y, x[5], a);
            a = fmaf(q1.z, x[6], a); a = fmaf(q1.w, x[7], a);
            sc[hh] = a;
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        sc[hh] += xor32(sc[hh]);
        if (tok >= nv) sc[hh] = -INFINITY;
      }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float mx = sc[hh];
#pragma unroll
        for (int o2 = 16; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
        const float mn = fmaxf(m[hh], mx);
        const float alpha = exp2f(m[hh] - mn);
        const float pe = exp2f(sc[hh] - mn);
        m[hh] = mn;
        lsum[hh] = lsum[hh] * alpha + (hf == 0 ? pe : 0.f);
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[hh][c] *= alpha;
        if (hf == 0) wp[wave][hh][tok] = pe;
      }
      wave_lds_sync();
#pragma unroll 1
      for (int t = 0; t < nv; ++t) {
        const int64_t slot = (t0 + t) % p.ring_slots;
        const uint8_t* row = slab + p.ring_base + (p.ring_slots + slot) * D * ib;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float x = load_in(row, lane * CPL + c, p.in_bf16);
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) o[hh][c] = fmaf(wp[wave][hh][t], x, o[hh][c]);
        }
      }
      wave_lds_sync();
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float l_ = lsum[hh];
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) l_ += __shfl_xor(l_, o2, 64);
#pragma unroll
      for (int c = 0; c < CPL; ++c) red[wave][hh][2 + lane * CPL + c] = o[hh][c];
      if (lane == 0) {
        red[wave][hh][0] = m[hh];
        red[wave][hh][1] = l_;
      }
    }
    __syncthreads();
  }
  __syncthreads();

  // ---- combine the waves; write the output or this block's partial ---------
  for (int i = tid; i < HG * D; i += kThreads) {
    const int hh = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[w][hh][0]);
    float so = 0.f, sl = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = exp2f(red[w][hh][0] - M);   // idle wave: m = -inf -> 0
      so = fmaf(e, red[w][hh][2 + c], so);
      sl = fmaf(e, red[w][hh][1], sl);
    }
    const int hq = h * HG + hh;
    if (p.splits == 1) {
      p.out[(static_cast<int64_t>(b) * p.q_heads + hq) * D + c] = so / sl;
    } else {
      float* part = p.partials + ((static_cast<int64_t>(b) * p.q_heads + hq) * p.splits + split) * (D + 2);
      part[2 + c] = so;
      if (c == 0) {
        part[0] = M;
        part[1] = sl;
      }
    }
  }
}

template <int BITS, int D>
hipError_t by_hg(const MfmaParams& p, int hg, int batch, hipStream_t st) {
  dim3 grid(p.splits, p.kv_heads, batch);
  switch (hg) {
    case 1: hipLaunchKernelGGL((kivi_mfma_kernel<BITS, D, 1>), grid, dim3(kThreads), 0, st, p); break;
    case 2: hipLaunchKernelGGL((kivi_mfma_kernel<BITS, D, 2>), grid, dim3(kThreads), 0, st, p); break;
    case 4: hipLaunchKernelGGL((kivi_mfma_kernel<BITS, D, 4>), grid, dim3(kThreads), 0, st, p); break;
    default: hipLaunchKernelGGL((kivi_mfma_kernel<BITS, D, 8>), grid, dim3(kThreads), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t by_d(const MfmaParams& p, int d, int hg, int batch, hipStream_t st) {
  switch (d) {
    case 64: return by_hg<BITS, 64>(p, hg, batch, st);
    case 128: return by_hg<BITS, 128>(p, hg, batch, st);
    default: return by_hg<BITS, 256>(p, hg, batch, st);
  }
}

}  // namespace

bool mfma_path(const Geometry& g) {
  return g.scheme == KVQ_KIVI && (g.bits == 2 || g.bits == 4) && g.d >= 64 && g.rope == 0.0;
}

MfmaPlan mfma_plan(const Geometry& g, int64_t tokens, int32_t requested) {
  MfmaPlan pl{};
  const int64_t q = kivi_quantised(tokens, g.residual);
  pl.pages = static_cast<int32_t>(q / kPage);
  pl.chunks = static_cast<int32_t>((tokens - q + kPage - 1) / kPage);
  if (pl.pages > 0) {
    int64_t s;
    if (requested > 0) {
      s = requested;
    } else {
      const int64_t units = static_cast<int64_t>(g.batch) * g.kv_heads;
      s = (1024 + units - 1) / units;
      const int64_t cap = (pl.pages + 7) / 8;
      if (s > cap) s = cap;
    }
    if (s > pl.pages) s = pl.pages;
    pl.page_splits = static_cast<int32_t>(s < 1 ? 1 : s);
  }
  pl.ring_splits = (pl.chunks + 7) / 8;
  // bound on ring blocks over every T (keeps the workspace size monotone)
  const int64_t max_chunks = (static_cast<int64_t>(g.residual) + 2 * kPage - 1) / kPage;
  pl.ring_splits_max = static_cast<int32_t>((max_chunks + 7) / 8);
  return pl;
}

hipError_t launch_kivi_mfma(const DecodeArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const MfmaPlan pl = mfma_plan(g, a.tokens, a.requested_splits);
  MfmaParams p{};
  p.layer_base = a.layer_base;
  p.q = static_cast<const uint8_t*>(a.q);
  p.out = a.out;
  p.partials = reinterpret_cast<float*>(a.workspace + workspace_partials_offset(g));
  p.slab_bytes = g.slab_bytes;
  p.page_bytes = g.page_bytes;
  p.ring_base = g.pages_per_slab * g.page_bytes;
  p.ring_slots = g.ring_slots;
  p.T = a.tokens;
  p.q_tokens = static_cast<int64_t>(pl.pages) * kPage;
  p.n_pages = pl.pages;
  p.n_chunks = pl.chunks;
  p.page_splits = pl.page_splits;
  p.splits = pl.page_splits + pl.ring_splits;
  p.kv_heads = g.kv_heads;
  p.q_heads = g.q_heads;
  p.off_ks = g.off_ks;
  p.off_kz = g.off_kz;
  p.off_vc = g.off_vc;
  p.off_vs = g.off_vs;
  p.off_vz = g.off_vz;
  p.q_bf16 = a.q_dtype == KVQ_BF16;
  p.in_bf16 = g.in_bytes == 2;
  p.qscale = a.sm_scale * kLog2e;
  hipError_t e = g.bits == 2 ? by_d<2>(p, g.d, g.hg, g.batch, st) : by_d<4>(p, g.d, g.hg, g.batch, st);
  if (e != hipSuccess) return e;
  if (p.splits > 1) return launch_merge(p.partials, p.out, g.batch * g.q_heads, p.splits, g.d, st);
  return hipSuccess;
}

}  // namespace kvq
