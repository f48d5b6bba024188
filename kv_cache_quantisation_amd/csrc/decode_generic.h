// The generic (vector-ALU) decode kernel, shared by the translation units that
// instantiate it for the scheme families (decode_kivi.hip: KIVI at 2/4/8 bits;
// decode_kivi3.hip: KIVI with 3-bit codes; decode_other.hip: symmetric, FP8
// and bfloat16 caches), so that they compile in parallel. decode.hip chooses
// the kernel for a call.
//
// Decode attention straight from the packed cache.
//
// out[b][h] = sum_t p_t V^_t with p = softmax(sm_scale q[b][h] . K^_t) over all
// cached tokens ("Quantizing the KV cache", going deeper: "Why values per
// token"); K^, V^ are the dequantised cache; query head h reads KV head
// h / (q_heads/kv_heads) (grouped-query attention, same page). With a rotary
// base the dequantised key at position t and the query at position T-1 are
// rotated (KVQuant Summary: keys cached before RoPE).
//
// Work split: for each (sequence, KV head) the pages (32 tokens each) and, for
// KIVI, the residual-ring chunks (32 tokens each) form a list of work items.
// The list is cut into `splits` contiguous ranges, one block of 4 waves per
// range; waves take items round-robin. Each wave keeps an online softmax
// (running max m, running sum l, unnormalised output o) for the GQA group of
// query heads; the waves are combined in LDS and the block writes one partial
// (m, l, o). The last block of a (sequence, KV head) to finish (an arrival
// counter in the workspace) merges the partials of every query row of that
// sequence: M = max m_s, out = sum 2^(m_s-M) o_s / sum 2^(m_s-M) l_s. Scores
// are kept in the log2 domain (the query is pre-scaled by sm_scale*log2(e)).
//
// Folding the scales out of the inner loops:
//   KIVI keys:   q.k^ = sum_c (q_c s_c) code_tc + sum_c q_c z_c  (per page)
//   KIVI values: sum_t p_t (code_tc s_t + z_t) = sum_t (p_t s_t) code_tc + sum_t p_t z_t
//   SYM:         q.k^ = s_t sum_c q_c code_tc;   values: p_t s_t
//   FP8:         the per-head key scale goes into q, the value scale into out.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_merge.h"
#include "kvq_wave.h"

namespace kvq {
namespace gen {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const uint8_t* layer_base;
  const uint8_t* q;
  const float* k_scale;
  const float* v_scale;
  float* out;
  float* partials;
  int* counters;        // one per (sequence, KV head), zero between calls
  int64_t slab_bytes, page_bytes, ring_base, ring_slots;
  int64_t T, q_tokens;  // cached tokens; tokens held in pages
  const int64_t* seq_tokens;   // ragged batch: per-sequence token counts (device), or null
  int32_t n_pages, items, splits;
  int32_t residual;            // R (the flush plan of a ragged KIVI sequence)
  int32_t nq;                  // queries per sequence (rows b * nq + i; 1 = one query)
  int32_t kv_heads, q_heads;
  int32_t off_kc, off_ks, off_kz, off_vc, off_vs, off_vz;
  int32_t q_bf16, in_bf16;
  float qscale;         // sm_scale * log2(e)
  double rope_theta;    // 0 = off
  int32_t outliers;     // KIVI dense-and-sparse pages: side matrix offsets below
  int32_t off_ko, off_vo, off_ki, off_vi;
  PageMap pm;           // pages and rings of the layer (slab or paged)
};

template <int BITS>
__device__ __forceinline__ float ucode(uint32_t w, int j) {
  return static_cast<float>((w >> (j * BITS)) & ((1u << BITS) - 1u));
}

template <int BITS>
__device__ __forceinline__ float scode(uint32_t w, int j) {
  const int32_t v = static_cast<int32_t>(w << (32 - (j + 1) * BITS)) >> (32 - BITS);
  return static_cast<float>(v);
}

// Field i of a packed run of B-bit fields that may straddle words (3-bit
// codes): read through a 64-bit window. The word after the field's first one
// is always inside the page (a code run is followed by its scales).
template <int B>
__device__ __forceinline__ uint32_t field_at(const uint32_t* run, int i) {
  const int bit = i * B, w = bit >> 5;
  const uint64_t v = (static_cast<uint64_t>(run[w + 1]) << 32) | run[w];
  return static_cast<uint32_t>(v >> (bit & 31)) & ((1u << B) - 1u);
}

// Value of a 3-bit code under the scheme's code type (KIVI unsigned, SYM
// two's complement).
template <int SCHEME>
__device__ __forceinline__ float code3_value(uint32_t f) {
  if constexpr (SCHEME == KVQ_SYM_TOKEN) return static_cast<float>(static_cast<int32_t>(f << 29) >> 29);
  else return static_cast<float>(f);
}

// Value of the j-th field of word w under the scheme's code type.
template <int SCHEME, int BITS>
__device__ __forceinline__ float code_value(uint32_t w, int j) {
  if constexpr (SCHEME == KVQ_KIVI) return ucode<BITS>(w, j);
  else if constexpr (SCHEME == KVQ_SYM_TOKEN) return scode<BITS>(w, j);
  else if constexpr (SCHEME == KVQ_FP8_E4M3) return e4m3_decode((w >> (8 * j)) & 0xFFu);
  else if constexpr (SCHEME == KVQ_FP8_E5M2) return e5m2_decode((w >> (8 * j)) & 0xFFu);
  else return __uint_as_float(j ? (w & 0xFFFF0000u) : (w << 16));   // bf16 field j
}

__device__ __forceinline__ float load_elem(const uint8_t* base, int64_t idx, int bf16) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

// Rotates (x0, x1) by 2*pi*frac(pos * w2pi).
__device__ __forceinline__ void rope_pair(float& x0, float& x1, int64_t pos, double w2pi) {
  const double turns = static_cast<double>(pos) * w2pi;
  const float f = static_cast<float>(turns - floor(turns));
  float s, c;
  sincospif(2.0f * f, &s, &c);
  const float y0 = x0 * c - x1 * s;
  const float y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

template <int SCHEME, int BITS, int VB, int D, int HG>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  // cache types of the key and of the value half (FP8K_SYMV / FP8K_KIVIV:
  // FP8 E4M3 keys, symmetric / KIVI per-token values; the other schemes use
  // one type for both)
  constexpr int KSCH = is_fp8_keys_mixed(SCHEME) ? KVQ_FP8_E4M3 : SCHEME;
  constexpr int VSCH = SCHEME == KVQ_FP8K_SYMV ? KVQ_SYM_TOKEN : SCHEME == KVQ_FP8K_KIVIV ? KVQ_KIVI : SCHEME;
  constexpr int CPL = D >= 64 ? D / 64 : 1;  // channels per lane in the P.V phase
  constexpr int LPC = D / CPL;                // lanes per token subset (64 or 32)
  constexpr int TSUB = 64 / LPC;              // token subsets (1, or 2 when D == 32)
  constexpr int TPS = kPage / TSUB;           // tokens per subset
  constexpr int HALF = D / 2;                 // channels per lane in the score phase
  constexpr int FPW = 32 / BITS;              // key fields per 32-bit word
  constexpr int FPWV = 32 / VB;               // value fields per 32-bit word (VB = value bits)
  constexpr int QROWS = HG > 2 ? HG : 2;
  constexpr int WQ = kWaves * QROWS * D;
  constexpr int RED = kWaves * HG * (D + 2);
  constexpr int SCRATCH = WQ > RED ? WQ : RED;

  __shared__ float qs[HG][D];
  __shared__ float scratch[SCRATCH];          // per-wave folded query / scales; later the combine
  __shared__ float wp[kWaves][HG][kPage];
  __shared__ double w2pi[D / 2];
  // dense-and-sparse pages (dynamic LDS, sized only when the cache has them),
  // per wave: oki[D] token of each key channel's outlier, okd[D] its value
  // (rotary keys) or its difference from the channel offset, voi[32] channel
  // of each value token's outlier, wpo[HG][32] the weight of its difference
  // from the token offset
  extern __shared__ float dyn_lds[];
  constexpr int OUT_LDS = 2 * D + kPage + HG * kPage;   // words per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tok = lane & 31, hf = lane >> 5;
  const int cs = lane % LPC, ts = lane / LPC;
  const int split = blockIdx.x, h = blockIdx.y;
  const int row = blockIdx.z;                 // query row: sequence b, query qi
  const int b = row / p.nq, qi = row - b * p.nq;
  const bool rope = p.rope_theta > 0.0;
  const uint8_t* ringp = p.pm.ring(b, h);
  float* wq = scratch + wave * QROWS * D;
  int* oki = reinterpret_cast<int*>(dyn_lds + wave * OUT_LDS);
  float* okd = dyn_lds + wave * OUT_LDS + D;
  int* voi = reinterpret_cast<int*>(dyn_lds + wave * OUT_LDS + 2 * D);
  float* wpo = dyn_lds + wave * OUT_LDS + 2 * D + kPage;   // [HG][32]
  // tokens this sequence holds (a ragged batch: its own fill level, and for
  // KIVI its own split between quantised pages and the ring)
  const int64_t fill = seq_len(p.seq_tokens, b, p.T);
  int64_t q_tokens = p.q_tokens;
  if (p.seq_tokens) q_tokens = SCHEME == KVQ_KIVI ? kivi_quantised(fill, p.residual) : fill;
  // tokens this row attends to: all of them, or with several queries per
  // sequence (the last nq tokens are theirs) query qi sees [0, fill - nq + qi]
  const int64_t Tb = fill - (p.nq - 1 - qi);
  int32_t n_pages, items;
  if (SCHEME == KVQ_KIVI && Tb > q_tokens) {   // every page, then ring chunks
    n_pages = static_cast<int32_t>(q_tokens / kPage);
    items = n_pages + static_cast<int32_t>((Tb - q_tokens + kPage - 1) / kPage);
  } else {                                     // the pages it reaches, the last perhaps in part
    n_pages = static_cast<int32_t>((Tb + kPage - 1) / kPage);
    items = n_pages;
  }

  // ---- stage the GQA group's query: rotate at T-1, scale ----------------------
  if (rope) {
    for (int i = tid; i < D / 2; i += kThreads)
      w2pi[i] = pow(p.rope_theta, -2.0 * i / D) * 0.15915494309189535;  // omega / (2 pi)
    __syncthreads();
  }
  {
    const float ks_h = is_fp8(KSCH) ? p.k_scale[h] : 1.0f;
    const float mult = p.qscale * ks_h;
    for (int i = tid; i < HG * D / 2; i += kThreads) {
      const int g = i / (D / 2), pr = i % (D / 2);
      const int64_t base = (static_cast<int64_t>(row) * p.q_heads + h * HG + g) * D + 2 * pr;
      float x0 = load_elem(p.q, base, p.q_bf16);
      float x1 = load_elem(p.q, base + 1, p.q_bf16);
      if (rope) {
        const double ang = static_cast<double>(Tb - 1) * (w2pi[pr] * 6.283185307179586);
        const double sn = sin(ang), cn = cos(ang);
        const double y0 = x0 * cn - x1 * sn, y1 = x0 * sn + x1 * cn;
        x0 = static_cast<float>(y0);
        x1 = static_cast<float>(y1);
      }
      qs[g][2 * pr] = x0 * mult;
      qs[g][2 * pr + 1] = x1 * mult;
    }
  }
  __syncthreads();

  // ---- item range of this split -------------------------------------------
  const int i0 = static_cast<int>(static_cast<int64_t>(split) * items / p.splits);
  const int i1 = static_cast<int>(static_cast<int64_t>(split + 1) * items / p.splits);
  const int rounds = (i1 - i0 + kWaves - 1) / kWaves;

  float m[HG], l_l[HG], z_l[HG], o[HG][CPL];
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    m[g] = -INFINITY;
    l_l[g] = 0.f;
    z_l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[g][c] = 0.f;
  }

  for (int r = 0; r < rounds; ++r) {
    const int item = i0 + r * kWaves + wave;
    const bool active = item < i1;
    const bool is_page = item < n_pages;
    // (the block table is read only for pages this wave takes)
    const uint8_t* pg = active && is_page ? p.pm.page(b, h, item) : ringp;
    const int64_t t_first = is_page ? static_cast<int64_t>(item) * kPage
                                    : q_tokens + static_cast<int64_t>(item - n_pages) * kPage;
    const int n_valid = static_cast<int>(Tb - t_first < kPage ? Tb - t_first : kPage);

    __syncthreads();
    // ---- prologue: per-page key scales ----------------------------------------
    float bias[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) bias[g] = 0.f;
    if (active && is_page && SCHEME == KVQ_KIVI) {
      const float* ksp = reinterpret_cast<const float*>(pg + p.off_ks);
      const float* kzp = reinterpret_cast<const float*>(pg + p.off_kz);
      for (int c = lane; c < D; c += 64) {
        const float s = ksp[c], z = kzp[c];
        if (p.outliers) {   // the channel's outlier: its token, and what it adds
          oki[c] = pg[p.off_ki + c];
          const float ko = reinterpret_cast<const float*>(pg + p.off_ko)[c];
          okd[c] = rope ? ko : ko - z;
        }
        if (rope) {
          wq[c] = s;
          wq[D + c] = z;
        } else {
#pragma unroll
          for (int g = 0; g < HG; ++g) {
            const float qv = qs[g][c];
            wq[g * D + c] = qv * s;
            bias[g] = fmaf(qv, z, bias[g]);
          }
        }
      }
      if (!rope) {
#pragma unroll
        for (int g = 0; g < HG; ++g) bias[g] = wave_sum(bias[g]);
      }
    }
    __syncthreads();

    // ---- scores: lane = (token, channel half) ----------------------------------
    float score[HG];
    if (active) {
      float acc[HG];
#pragma unroll
      for (int g = 0; g < HG; ++g) acc[g] = 0.f;
      const bool valid = tok < n_valid;
      if (is_page) {
        // KIVI keys without rotation use the per-page folded query
        const float* qsrc = (SCHEME == KVQ_KIVI && !rope) ? wq : &qs[0][0];
        constexpr int NWORD = D * BITS / 64;   // words per half row
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(pg + p.off_kc) +
                             tok * (D * BITS / 32) + hf * NWORD;
        float kst = 1.0f;
        if constexpr (KSCH == KVQ_SYM_TOKEN)
          kst = reinterpret_cast<const float*>(pg + p.off_ks)[tok];
        if constexpr (BITS == 3) {
          // 3-bit fields straddle words: 8 channels at a time from the row
          const uint32_t* krow = reinterpret_cast<const uint32_t*>(pg + p.off_kc) + tok * (D * 3 / 32);
          for (int c0 = hf * HALF; c0 < hf * HALF + HALF; c0 += 8) {
            float kv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] = code3_value<KSCH>(field_at<3>(krow, c0 + j));
            if (rope) {
              if constexpr (SCHEME == KVQ_KIVI) {
#pragma unroll
                for (int j = 0; j < 8; ++j) kv[j] = kv[j] * wq[c0 + j] + wq[D + c0 + j];
                if (p.outliers) {
#pragma unroll
                  for (int j = 0; j < 8; ++j) kv[j] = oki[c0 + j] == tok ? okd[c0 + j] : kv[j];
                }
              }
#pragma unroll
              for (int j = 0; j < 8; j += 2)
                rope_pair(kv[j], kv[j + 1], t_first + tok, w2pi[(c0 + j) / 2]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
              for (int g = 0; g < HG; ++g)
                acc[g] = fmaf(qsrc[g * D + c0 + j], kv[j], acc[g]);
            }
          }
        } else {
#pragma unroll
        for (int wi = 0; wi < NWORD; ++wi) {
          const uint32_t w = kw[wi];
          const int c0 = hf * HALF + wi * FPW;
          float kv[FPW];
#pragma unroll
          for (int j = 0; j < FPW; ++j) kv[j] = code_value<KSCH, BITS>(w, j);
          if (rope) {
            if constexpr (SCHEME == KVQ_KIVI) {
#pragma unroll
              for (int j = 0; j < FPW; ++j) kv[j] = kv[j] * wq[c0 + j] + wq[D + c0 + j];
              if (p.outliers) {   // the side matrix's exact value at its position
#pragma unroll
                for (int j = 0; j < FPW; ++j) kv[j] = oki[c0 + j] == tok ? okd[c0 + j] : kv[j];
              }
            }
#pragma unroll
            for (int j = 0; j < FPW; j += 2)
              rope_pair(kv[j], kv[j + 1], t_first + tok, w2pi[(c0 + j) / 2]);
          }
#pragma unroll
          for (int j = 0; j < FPW; ++j) {
#pragma unroll
            for (int g = 0; g < HG; ++g)
              acc[g] = fmaf(qsrc[g * D + c0 + j], kv[j], acc[g]);
          }
        }
        }   // 3-bit / word-aligned fields
#pragma unroll
        for (int g = 0; g < HG; ++g) acc[g] *= kst;
        if (SCHEME == KVQ_KIVI && p.outliers && !rope) {
          // moved key values: code 0 gave q z; add q (outlier - z)
          for (int c = hf * HALF; c < hf * HALF + HALF; ++c) {
            if (oki[c] == tok) {
#pragma unroll
              for (int g = 0; g < HG; ++g) acc[g] = fmaf(qs[g][c], okd[c], acc[g]);
            }
          }
        }
      } else {
        // residual ring: exact input-dtype rows
        const int64_t t = t_first + tok;
        if (valid) {
          const int64_t slot = t % p.ring_slots;
          const uint8_t* row = ringp + slot * D * (p.in_bf16 ? 2 : 4);
          for (int c = hf * HALF; c < hf * HALF + HALF; c += 2) {
            float x0 = load_elem(row, c, p.in_bf16);
            float x1 = load_elem(row, c + 1, p.in_bf16);
            if (rope) rope_pair(x0, x1, t, w2pi[c / 2]);
#pragma unroll
            for (int g = 0; g < HG; ++g) acc[g] = fmaf(qs[g][c + 1], x1, fmaf(qs[g][c], x0, acc[g]));
          }
        }
      }
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        acc[g] += __shfl_xor(acc[g], 32, 64);
        score[g] = valid ? acc[g] + bias[g] : -INFINITY;
      }

      // ---- online softmax --------------------------------------------------
      float vsc = 1.0f, vz = 0.0f, vdo = 0.0f;
      if (is_page && valid) {
        if constexpr (VSCH == KVQ_KIVI) {
          vsc = reinterpret_cast<const float*>(pg + p.off_vs)[tok];
          vz = reinterpret_cast<const float*>(pg + p.off_vz)[tok];
          if (SCHEME == KVQ_KIVI && p.outliers) {   // moved value: code 0 gave z; its channel gets (outlier - z)
            vdo = reinterpret_cast<const float*>(pg + p.off_vo)[tok] - vz;
            if (hf == 0) voi[tok] = pg[p.off_vi + tok];
          }
        } else if constexpr (VSCH == KVQ_SYM_TOKEN) {
          vsc = reinterpret_cast<const float*>(pg + p.off_vs)[tok];
        }
      }
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const float mn = fmaxf(m[g], half_max(score[g]));
        const float alpha = exp2f(m[g] - mn);
        const float pe = exp2f(score[g] - mn);
        m[g] = mn;
        l_l[g] = l_l[g] * alpha + (hf == 0 ? pe : 0.f);
        z_l[g] = z_l[g] * alpha + (hf == 0 ? pe * vz : 0.f);
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[g][c] *= alpha;
        if (hf == 0) wp[wave][g][tok] = valid ? pe * vsc : 0.f;
        if (p.outliers && hf == 0) wpo[g * kPage + tok] = valid ? pe * vdo : 0.f;
      }
      if (p.outliers && hf == 0 && !(is_page && valid)) voi[tok] = -1;
    }
    __syncthreads();

    // ---- P.V: lane = (channel set, token subset) --------------------------------
    if (active) {
      if (is_page) {
        constexpr int COLW = kPage * VB / 32;     // words per channel column
        constexpr int SUBW = TPS * VB / 32;       // words per token subset
        if constexpr (VB == 3) {   // 3-bit fields straddle words
#pragma unroll
          for (int ci = 0; ci < CPL; ++ci) {
            const int c = cs * CPL + ci;
            const uint32_t* col = reinterpret_cast<const uint32_t*>(pg + p.off_vc) + c * COLW;
            for (int j = 0; j < TPS; ++j) {
              const int t = ts * TPS + j;
              const float cv = code3_value<VSCH>(field_at<3>(col, t));
#pragma unroll
              for (int g = 0; g < HG; ++g) o[g][ci] = fmaf(wp[wave][g][t], cv, o[g][ci]);
            }
          }
        } else {
        // FP8 values of the cache's open last page (fewer than 32 tokens) are
        // in token rows: the 4 codes of a word are gathered from 4 rows
        const bool vrows = (SCHEME == KVQ_FP8_E4M3 || SCHEME == KVQ_FP8_E5M2) && fill % kPage != 0 &&
                           item == fill / kPage;
#pragma unroll
        for (int ci = 0; ci < CPL; ++ci) {
          const int c = cs * CPL + ci;
          const uint32_t* vw = reinterpret_cast<const uint32_t*>(pg + p.off_vc) + c * COLW +
                               ts * SUBW;
#pragma unroll
          for (int wi = 0; wi < SUBW; ++wi) {
            uint32_t w;
            if (vrows) {
              const uint8_t* vr = pg + p.off_vc + static_cast<int64_t>(ts * TPS + wi * FPWV) * D + c;
              w = uint32_t(vr[0]) | (uint32_t(vr[D]) << 8) | (uint32_t(vr[2 * D]) << 16) |
                  (uint32_t(vr[3 * D]) << 24);
            } else {
              w = vw[wi];
            }
#pragma unroll
            for (int j = 0; j < FPWV; ++j) {
              const float cv = code_value<VSCH, VB>(w, j);
              const int t = ts * TPS + wi * FPWV + j;
#pragma unroll
              for (int g = 0; g < HG; ++g) o[g][ci] = fmaf(wp[wave][g][t], cv, o[g][ci]);
            }
          }
        }
        }   // 3-bit / word-aligned fields
        if (SCHEME == KVQ_KIVI && p.outliers) {
          for (int j = 0; j < TPS; ++j) {
            const int t = ts * TPS + j;
            const int oc = voi[t] - cs * CPL;   // outlier channel relative to this lane's
            if (oc >= 0 && oc < CPL) {
#pragma unroll
              for (int ci = 0; ci < CPL; ++ci) {
                if (ci == oc) {
#pragma unroll
                  for (int g = 0; g < HG; ++g) o[g][ci] += wpo[g * kPage + t];
                }
              }
            }
          }
        }
      } else {
        const int ib = p.in_bf16 ? 2 : 4;
        for (int j = 0; j < TPS; ++j) {
          const int tl = ts * TPS + j;
          if (tl >= n_valid) break;
          const int64_t slot = (t_first + tl) % p.ring_slots;
          const uint8_t* row = ringp + (p.ring_slots + slot) * D * ib;
#pragma unroll
          for (int ci = 0; ci < CPL; ++ci) {
            const float x = load_elem(row, cs * CPL + ci, p.in_bf16);
#pragma unroll
            for (int g = 0; g < HG; ++g) o[g][ci] = fmaf(wp[wave][g][tl], x, o[g][ci]);
          }
        }
      }
    }
  }

  // ---- combine the waves ----------------------------------------------------
  __syncthreads();
  float* red = scratch;  // [wave][g][D + 2]: m, l, o[D]
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    const float lw = wave_sum(l_l[g]);
    const float zw = wave_sum(z_l[g]);
    float* rw = red + (wave * HG + g) * (D + 2);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float v = o[g][c];
      if constexpr (TSUB == 2) v += __shfl_xor(v, 32, 64);
      if (ts == 0) rw[2 + cs * CPL + c] = v + zw;
    }
    if (lane == 0) {
      rw[0] = m[g];
      rw[1] = lw;
    }
  }
  __syncthreads();
  // several blocks per (sequence, KV head): count this block's arrival first;
  // the round trip overlaps the combination of the waves below
  __shared__ int last_block;
  const int unit = b * p.kv_heads + h;   // one arrival counter for every row of b
  int arrived = 0;
  if (p.splits > 1 && tid == 0) arrived = count_arrival(&p.counters[unit]);
  const float vsc_h = is_fp8(VSCH) ? p.v_scale[h] : 1.0f;
  constexpr int PER = (HG * D + kThreads - 1) / kThreads;
  float own_m[PER], own_l[PER], own_o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = tid + e * kThreads;
    own_m[e] = -INFINITY;
    own_l[e] = 0.f;
    own_o[e] = 0.f;
    if (i < HG * D) {
      const int g = i / D, c = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[(w * HG + g) * (D + 2)]);
      float so = 0.f, sl = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* rw = red + (w * HG + g) * (D + 2);
        const float ew = exp2_rel(rw[0], M);  // empty wave (or split): 0
        so = fmaf(ew, rw[2 + c], so);
        sl = fmaf(ew, rw[1], sl);
      }
      so *= vsc_h;
      if (p.splits == 1) p.out[(static_cast<int64_t>(row) * p.q_heads + h * HG + g) * D + c] = so / sl;
      own_m[e] = M;
      own_l[e] = sl;
      own_o[e] = so;
    }
  }
  if (p.splits == 1) return;

  // ---- the last of the nq * splits blocks of (b, h) to arrive merges --------
  if (tid == 0) last_block = arrived == p.nq * p.splits - 1;
  __syncthreads();
  float* part_rh = p.partials + (static_cast<int64_t>(row) * p.q_heads + h * HG) * p.splits * (D + 2);
  if (!last_block) {
    store_partial<D, HG, kThreads>(part_rh, p.splits, split, own_m, own_l, own_o, tid);
    return;
  }
  merge_partials<D, HG, kThreads>(p.partials, p.out, &p.counters[unit], p.q_heads, p.splits, p.nq, b, h,
                                  row, split, own_m, own_l, own_o, tid);
}

template <int SCHEME, int BITS, int VB, int D, int HG>
hipError_t launch(const DecodeParams& p, int batch, hipStream_t st) {
  dim3 grid(p.splits, p.kv_heads, batch * p.nq);
  const size_t dyn = p.outliers ? kWaves * (2 * D + kPage + HG * kPage) * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_split_kernel<SCHEME, BITS, VB, D, HG>), grid, dim3(kThreads), dyn, st, p);
  return hipGetLastError();
}

template <int SCHEME, int BITS, int VB, int D>
hipError_t by_hg(const DecodeParams& p, int hg, int batch, hipStream_t st) {
  switch (hg) {
    case 1: return launch<SCHEME, BITS, VB, D, 1>(p, batch, st);
    case 2: return launch<SCHEME, BITS, VB, D, 2>(p, batch, st);
    case 4: return launch<SCHEME, BITS, VB, D, 4>(p, batch, st);
    default: return launch<SCHEME, BITS, VB, D, 8>(p, batch, st);
  }
}

// VB: bits of the value codes (KIVI may store values narrower than keys)
template <int SCHEME, int BITS, int VB = BITS>
hipError_t by_d(const DecodeParams& p, int d, int hg, int batch, hipStream_t st) {
  switch (d) {
    case 32: return by_hg<SCHEME, BITS, VB, 32>(p, hg, batch, st);
    case 64: return by_hg<SCHEME, BITS, VB, 64>(p, hg, batch, st);
    case 128: return by_hg<SCHEME, BITS, VB, 128>(p, hg, batch, st);
    default: return by_hg<SCHEME, BITS, VB, 256>(p, hg, batch, st);
  }
}


// Launchers of the scheme families (one translation unit each).
hipError_t run_kivi(const DecodeParams& p, const Geometry& g, hipStream_t st);
hipError_t run_kivi3(const DecodeParams& p, const Geometry& g, hipStream_t st);
hipError_t run_other(const DecodeParams& p, const Geometry& g, hipStream_t st);
hipError_t run_mixed(const DecodeParams& p, const Geometry& g, hipStream_t st);

}  // namespace gen
}  // namespace kvq
