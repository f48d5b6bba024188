// Quantize-append kernels.
//
// KIVI ("Quantizing the KV cache", going deeper: Q_b and s; "Keys and values
// are shaped differently"; KIVI How It Works): when the unquantised window
// holds R+32 tokens, its oldest 32 are encoded as one page -- keys per channel
// over the 32 tokens, values per token over the head's channels -- and the
// newest tokens are copied bit-exactly into the residual ring. A page being
// encoded may draw tokens from the ring (appended by earlier calls) and from
// this call's input, so the flush runs before the ring is overwritten: two
// launches in stream order.
//
// SYM_TOKEN ("Quantising the Cache.", Workshop), FP8 E4M3 / E5M2 ("Quantizing
// the KV cache", FP8 KV cache with per-head scales) and the bfloat16 cache:
// every new token is encoded on arrival into the page that holds it. Value
// codes are channel-major inside a page; SYM_TOKEN codes narrower than a byte
// update a partially filled page with read-modify-write of the words that
// carry the new tokens' fields (each word owned by one thread), byte-aligned
// codes are stored whole.
//
// All encoding arithmetic is fp32 with IEEE division and rintf (ties to
// even); the library is compiled with -ffp-contract=off so no FMA is formed.
#include <hip/hip_runtime.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;

struct AppendParams {
  uint8_t* layer_base;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const float* k_scale;
  const float* v_scale;
  int64_t slab_bytes, page_bytes, ring_base;  // ring_base = P * page_bytes
  int64_t past, n;                            // tokens held before the call, appended
  int64_t stride;                             // input rows per sequence (n, or the ragged bound)
  const int64_t* seq_past;                    // ragged batch: per-sequence past and new
  const int64_t* seq_new;                     //   counts (device), or null
  int64_t capacity;                           // max_tokens
  int32_t residual;                           // R (KIVI)
  int64_t ring_slots;
  int32_t kv_heads;
  int32_t off_kc, off_ks, off_kz, off_vc, off_vs, off_vz;
  int32_t outliers;                           // KIVI dense-and-sparse pages (0 or 1)
  int32_t off_ko, off_vo, off_ki, off_vi;     // their side matrix
  PageMap pm;                                 // pages and rings of the layer (slab or paged)
};

// Tokens sequence b held before the call and tokens it appends: the uniform
// counts, or its own counts of a ragged batch, clamped so that every write
// stays in its slab (0 <= past <= capacity, 0 <= n <= min(stride, capacity - past)).
__device__ __forceinline__ void seq_counts(const AppendParams& p, int b, int64_t& past, int64_t& n) {
  past = p.past;
  n = p.n;
  if (p.seq_past) {
    const int64_t ps = p.seq_past[b], ns = p.seq_new[b];
    past = ps < 0 ? 0 : (ps > p.capacity ? p.capacity : ps);
    const int64_t room = p.capacity - past < p.stride ? p.capacity - past : p.stride;
    n = ns < 0 ? 0 : (ns > room ? room : ns);
  }
}

// Places a B-bit code as field i of a run of 32 fields held in B words (3-bit
// fields straddle words): or-ed into w, its bits recorded in m.
template <int B>
__device__ __forceinline__ void put_field(uint32_t (&w)[B], uint32_t (&m)[B], int i, uint32_t code) {
  constexpr uint32_t F = (1u << B) - 1u;
  const int bit = i * B, k = bit >> 5, sh = bit & 31;
  w[k] |= code << sh;
  m[k] |= F << sh;
  if (sh + B > 32) {
    w[k + 1] |= code >> (32 - sh);
    m[k + 1] |= F >> (32 - sh);
  }
}

// Widens one 16-byte chunk of a token row (bf16 or f32) into an fp32 LDS row.
template <int IB>
__device__ __forceinline__ void stage_chunk(const uint4& v, float* dst, int chunk) {
  if constexpr (IB == 2) {
    float f[8];
    unpack_bf16x8(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[chunk * 8 + i] = f[i];
  } else {
    dst[chunk * 4 + 0] = __uint_as_float(v.x);
    dst[chunk * 4 + 1] = __uint_as_float(v.y);
    dst[chunk * 4 + 2] = __uint_as_float(v.z);
    dst[chunk * 4 + 3] = __uint_as_float(v.w);
  }
}

// ---- KIVI: encode one 32-token page per block --------------------------------
// grid = (pages to flush, kv_heads, batch). The page's 32 key and value rows
// are staged in LDS in the input dtype (padded rows); every thread then takes
// part in the statistics (several threads per key channel / value token,
// combined with lane shuffles) and in the codes (one or more packed words per
// thread), where each quotient comes from a reciprocal with an exact fallback.
// OUT: dense-and-sparse pages (a template parameter, so that dense pages
// compile exactly as without the feature)
template <int D, int KB, int VB, int IB, bool OUT>
__global__ __launch_bounds__(kThreads) void kivi_flush_kernel(AppendParams p) {
  constexpr float kLevelsK = float((1 << KB) - 1);   // key / value code levels
  constexpr float kLevelsV = float((1 << VB) - 1);
  constexpr int FPWK = 32 / KB;               // fields per 32-bit word
  constexpr int FPWV = 32 / VB;
  constexpr int ROW = D * IB;                 // bytes per input row
  constexpr int PITCH = ROW + 16;             // padded LDS row
  constexpr int CHUNKS = ROW / 16;            // 16-byte chunks per row
  constexpr int TPC = kThreads / D > 1 ? kThreads / D : 1;   // threads per key channel
  constexpr int RPT = kPage / TPC;            // rows per thread (key statistics)
  constexpr int TPT = kThreads / kPage;       // threads per value token (8)
  constexpr int CPT = D / TPT;                // channels per thread (value statistics)
  static_assert(TPC <= 8 && (TPC & (TPC - 1)) == 0, "key statistics lane groups");
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kPage * PITCH];   // K rows, V rows
  __shared__ __attribute__((aligned(16))) float k_mn[D], k_s[D], k_r[D], v_mn[kPage], v_s[kPage], v_r[kPage];
  // dense-and-sparse pages: the token of each key channel's outlier and the
  // channel of each value token's outlier
  __shared__ int k_oi[D], v_oi[kPage];

  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  int64_t past, n;
  seq_counts(p, b, past, n);
  // pages this sequence flushes: [q(past), q(past + n)) / 32
  const int64_t page = kivi_quantised(past, p.residual) / kPage + blockIdx.x;
  if (page >= kivi_quantised(past + n, p.residual) / kPage) return;   // whole block
  uint8_t* pg = p.pm.page(b, h, page);
  const uint8_t* ringp = p.pm.ring(b, h);

  auto elem = [&](int which, int r, int c) -> float {
    const uint8_t* row = tile[which] + r * PITCH;
    if constexpr (IB == 2) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[c]);
    else return reinterpret_cast<const float*>(row)[c];
  };

  // 1. stage the page's 32 key and value rows (ring for tokens < past, else
  //    input): every load of the thread is issued before the first LDS write
  //    (no branch between them: each row's source is a select)
  constexpr int NCH = 2 * kPage * CHUNKS;
  static_assert(NCH % kThreads == 0, "whole chunks per thread");
  constexpr int SPT = NCH / kThreads;          // 16-byte chunks per thread
  const int64_t t_page = page * kPage;
  const int slots = static_cast<int>(p.ring_slots);
  const int s0 = static_cast<int>(t_page % p.ring_slots);
  {
    uint4 chunk[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid + k * kThreads;
      const int which = i / (kPage * CHUNKS);   // 0 = K, 1 = V
      const int r = (i / CHUNKS) % kPage;
      const int64_t t = t_page + r;
      const int slot = s0 + r >= slots ? s0 + r - slots : s0 + r;
      const uint8_t* ring = ringp + (static_cast<int64_t>(which) * p.ring_slots + slot) * ROW;
      const int64_t j = t >= past ? t - past : 0;
      const uint8_t* in = (which ? p.v_new : p.k_new) +
                          ((static_cast<int64_t>(b) * p.stride + j) * p.kv_heads + h) * ROW;
      chunk[k] = *reinterpret_cast<const uint4*>((t < past ? ring : in) + (i % CHUNKS) * 16);
    }
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int i = tid + k * kThreads;
      const int which = i / (kPage * CHUNKS);
      const int r = (i / CHUNKS) % kPage;
      *reinterpret_cast<uint4*>(tile[which] + r * PITCH + (i % CHUNKS) * 16) = chunk[k];
    }
  }
  __syncthreads();

  // Largest magnitude over a lane group's candidates (index lo, magnitude a):
  // the larger one, the lower index among equal magnitudes.
  auto argmax_abs = [](float& a, int& lo, int lanes) {
    for (int m = 1; m < lanes; m <<= 1) {
      const float oa = __shfl_xor(a, m, 64);
      const int ol = __shfl_xor(lo, m, 64);
      if (oa > a || (oa == a && ol < lo)) {
        a = oa;
        lo = ol;
      }
    }
  };

  // 2a. key statistics per channel over the 32 tokens (TPC lanes per channel);
  //     dense-and-sparse pages first move each channel's largest |x| out
  for (int c0 = 0; c0 < D; c0 += kThreads / TPC) {
    const int c = c0 + tid / TPC, part = tid % TPC;
    int oi = -1;   // token of this channel's outlier
    if constexpr (OUT) {
      float best = -1.0f;
      int bi = 0;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const float a = fabsf(elem(0, part * RPT + r, c));
        if (a > best) {
          best = a;
          bi = part * RPT + r;
        }
      }
      argmax_abs(best, bi, TPC);
      oi = bi;
    }
    float mn = INFINITY, mx = -INFINITY;
    if (c < D) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const float x = elem(0, part * RPT + r, c);
        if (part * RPT + r != oi) {
          mn = fminf(mn, x);
          mx = fmaxf(mx, x);
        }
      }
    }
#pragma unroll
    for (int m = 1; m < TPC; m <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, m, 64));
      mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    if (c < D && part == 0) {
      mn = mn + 0.0f;                          // -0 -> +0
      const float s = (mx - mn) / kLevelsK;
      k_mn[c] = mn;
      k_s[c] = s;
      k_r[c] = quant_rcp_prep(s);
      if constexpr (OUT) k_oi[c] = oi;
      reinterpret_cast<float*>(pg + p.off_ks)[c] = s;
      reinterpret_cast<float*>(pg + p.off_kz)[c] = mn;
      if constexpr (OUT) {
        reinterpret_cast<float*>(pg + p.off_ko)[c] = elem(0, oi, c);   // exact input value
        pg[p.off_ki + c] = static_cast<uint8_t>(oi);
      }
    }
  }
  // 2b. value statistics per token over the D channels (8 lanes per token)
  {
    const int r = tid / TPT, part = tid % TPT;
    int oi = -1;   // channel of this token's outlier
    if constexpr (OUT) {
      float best = -1.0f;
      int bi = 0;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const float a = fabsf(elem(1, r, part * CPT + i));
        if (a > best) {
          best = a;
          bi = part * CPT + i;
        }
      }
      argmax_abs(best, bi, TPT);
      oi = bi;
    }
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const float x = elem(1, r, part * CPT + i);
      if (part * CPT + i != oi) {
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
    }
#pragma unroll
    for (int m = 1; m < TPT; m <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, m, 64));
      mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    if (part == 0) {
      mn = mn + 0.0f;
      const float s = (mx - mn) / kLevelsV;
      v_mn[r] = mn;
      v_s[r] = s;
      v_r[r] = quant_rcp_prep(s);
      if constexpr (OUT) v_oi[r] = oi;
      reinterpret_cast<float*>(pg + p.off_vs)[r] = s;
      reinterpret_cast<float*>(pg + p.off_vz)[r] = mn;
      if constexpr (OUT) {
        reinterpret_cast<float*>(pg + p.off_vo)[r] = elem(1, r, oi);   // exact input value
        pg[p.off_vi + r] = static_cast<uint8_t>(oi);
      }
    }
  }
  __syncthreads();

  // 3. codes. K rows: field f = token*D + channel. V cols: field f = channel*32 + token.
  //    Statistics and key elements of a word are read as vectors.
  constexpr int WORDSK = kPage * D * KB / 32;
  constexpr int WORDSV = kPage * D * VB / 32;
  uint32_t* kc = reinterpret_cast<uint32_t*>(pg + p.off_kc);
  uint32_t* vc = reinterpret_cast<uint32_t*>(pg + p.off_vc);
  auto load4 = [](const float* src, auto& dst) {   // all of dst, 16-byte aligned src
    constexpr int N = sizeof(dst) / sizeof(float);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(src)[i];
      dst[4 * i] = v.x;
      dst[4 * i + 1] = v.y;
      dst[4 * i + 2] = v.z;
      dst[4 * i + 3] = v.w;
    }
  };
  if constexpr (KB == 3) {
    // 3-bit K rows: groups of 32 fields (a token's 32 channels) in 3 words
    for (int gi = tid; gi < kPage * D / 32; gi += kThreads) {
      const int t = gi * 32 / D, c0 = gi * 32 % D;
      uint32_t wd[3] = {0u, 0u, 0u}, m[3] = {0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        uint32_t code = quant_asym_rcp(elem(0, t, c0 + j), k_mn[c0 + j], k_s + c0 + j,
                                       k_r[c0 + j], kLevelsK);
        if (OUT && k_oi[c0 + j] == t) code = 0u;
        put_field<3>(wd, m, j, code);
      }
      kc[3 * gi] = wd[0];
      kc[3 * gi + 1] = wd[1];
      kc[3 * gi + 2] = wd[2];
    }
  } else
  for (int w = tid; w < WORDSK; w += kThreads) {
    const int f0 = w * FPWK;
    const int t = f0 / D, c0 = f0 % D;
    float x[FPWK], mn[FPWK], rc[FPWK];
    const uint8_t* row = tile[0] + t * PITCH + c0 * IB;
    if constexpr (IB == 2) {
      if constexpr (FPWK >= 8) {
#pragma unroll
        for (int i = 0; i < FPWK / 8; ++i) unpack_bf16x8(reinterpret_cast<const uint4*>(row)[i], x + 8 * i);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(row);
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
      }
    } else {
      load4(reinterpret_cast<const float*>(row), x);
    }
    load4(k_mn + c0, mn);
    load4(k_r + c0, rc);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < FPWK; ++j)
      word |= quant_asym_rcp(x[j], mn[j], k_s + c0 + j, rc[j], kLevelsK) << (j * KB);
    if constexpr (OUT) {   // the moved values' fields hold code 0
#pragma unroll
      for (int j = 0; j < FPWK; ++j)
        if (k_oi[c0 + j] == t) word &= ~(((1u << KB) - 1u) << (j * KB));
    }
    kc[w] = word;
  }
  if constexpr (VB == 3) {
    // 3-bit V cols: a channel's 32 tokens in 3 words
    for (int c = tid; c < D; c += kThreads) {
      uint32_t wd[3] = {0u, 0u, 0u}, m[3] = {0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        uint32_t code = quant_asym_rcp(elem(1, t, c), v_mn[t], v_s + t, v_r[t], kLevelsV);
        if (OUT && v_oi[t] == c) code = 0u;
        put_field<3>(wd, m, t, code);
      }
      vc[3 * c] = wd[0];
      vc[3 * c + 1] = wd[1];
      vc[3 * c + 2] = wd[2];
    }
  } else
  for (int w = tid; w < WORDSV; w += kThreads) {
    const int f0 = w * FPWV;
    const int c = f0 / kPage, t0 = f0 % kPage;
    float mn[FPWV], rc[FPWV];
    load4(v_mn + t0, mn);
    load4(v_r + t0, rc);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < FPWV; ++j)
      word |= quant_asym_rcp(elem(1, t0 + j, c), mn[j], v_s + t0 + j, rc[j], kLevelsV) << (j * VB);
    if constexpr (OUT) {
#pragma unroll
      for (int j = 0; j < FPWV; ++j)
        if (v_oi[t0 + j] == c) word &= ~(((1u << VB) - 1u) << (j * VB));
    }
    vc[w] = word;
  }
}

// ---- KIVI: copy tokens [t0, past+n) of the input into their ring slots --------
// grid = (tokens, kv_heads, batch), one 16-byte chunk per thread
template <int D, int IB>
__global__ __launch_bounds__(64) void ring_write_kernel(AppendParams p) {
  constexpr int CHUNKS = D * IB / 16;
  const int h = blockIdx.y, b = blockIdx.z;
  int64_t past, n;
  seq_counts(p, b, past, n);
  // tokens [max(q(past + n), past), past + n) stay in the ring
  const int64_t q_new = kivi_quantised(past + n, p.residual);
  const int64_t t = (q_new > past ? q_new : past) + blockIdx.x;
  if (t >= past + n) return;
  const int64_t j = t - past;
  const int64_t row_bytes = static_cast<int64_t>(D) * IB;
  uint8_t* ringp = p.pm.ring(b, h);
  const int64_t slot = t % p.ring_slots;
  const int64_t in_off = ((static_cast<int64_t>(b) * p.stride + j) * p.kv_heads + h) * row_bytes;
  for (int i = threadIdx.x; i < 2 * CHUNKS; i += 64) {
    const int which = i / CHUNKS, c = i % CHUNKS;
    const uint8_t* src = (which ? p.v_new : p.k_new) + in_off + c * 16;
    uint8_t* dst = ringp + (which * p.ring_slots + slot) * row_bytes + c * 16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// ---- SYM_TOKEN: encode the new tokens of one page per block -------------------
// grid = (pages touched, kv_heads, batch). Codes narrower than a byte share
// 32-bit words across tokens, so the page's new rows are staged in LDS first.
// WITH_K false: the values only (keys in another cache type, written by
// another kernel). ASYM (values only): each value token encoded as KIVI
// encodes its values, unsigned codes over [min, max] with a per-token scale
// and offset, instead of the symmetric codes.
template <int D, int BITS, int IB, bool WITH_K = true, bool ASYM = false>
__global__ __launch_bounds__(kThreads) void token_append_kernel(AppendParams p) {
  static_assert(!(ASYM && WITH_K), "asymmetric codes for the value half only");
  constexpr int LD = D + 1;
  constexpr int FPW = 32 / BITS;
  constexpr int CHUNKS = D * IB / 16;
  constexpr uint32_t kMask = (1u << BITS) - 1u;  // BITS < 32
  constexpr float kQmax = float((1 << (BITS - 1)) - 1);
  constexpr float kLevels = float((1 << BITS) - 1);
  __shared__ float ktile[kPage * LD];
  __shared__ float vtile[kPage * LD];
  __shared__ float k_sc[kPage], v_sc[kPage], v_mn[kPage];

  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  int64_t past, n;
  seq_counts(p, b, past, n);
  const int64_t page = past / kPage + blockIdx.x;
  const int64_t end = past + n;
  if (n == 0 || page > (end - 1) / kPage) return;   // whole block
  const int lo = static_cast<int>((past > page * kPage ? past : page * kPage) - page * kPage);
  const int hi = static_cast<int>((end < page * kPage + kPage ? end : page * kPage + kPage) -
                                  page * kPage);
  uint8_t* pg = p.pm.page(b, h, page);
  const int64_t row_bytes = static_cast<int64_t>(D) * IB;

  // every load of the thread is issued before the first LDS write (threads
  // past the last chunk load chunk 0 again and do not store it)
  constexpr int HALVES = WITH_K ? 2 : 1;   // K and V rows, or V rows only
  constexpr int SPT = (HALVES * kPage * CHUNKS + kThreads - 1) / kThreads;   // chunks per thread, at most
  uint4 chunk[SPT];
  const int nch = HALVES * (hi - lo) * CHUNKS;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int i = tid + k * kThreads < nch ? tid + k * kThreads : 0;
    const int which = WITH_K ? i / ((hi - lo) * CHUNKS) : 1;
    const int r = lo + (i / CHUNKS) % (hi - lo);
    const int64_t j = page * kPage + r - past;
    const uint8_t* src = (which ? p.v_new : p.k_new) +
                         ((static_cast<int64_t>(b) * p.stride + j) * p.kv_heads + h) * row_bytes;
    chunk[k] = *reinterpret_cast<const uint4*>(src + (i % CHUNKS) * 16);
  }
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int i = tid + k * kThreads;
    if (i < nch) {
      const int which = WITH_K ? i / ((hi - lo) * CHUNKS) : 1;
      const int r = lo + (i / CHUNKS) % (hi - lo);
      const int c = i % CHUNKS;
      stage_chunk<IB>(chunk[k], (which ? vtile : ktile) + r * LD, c);
    }
  }
  __syncthreads();

  // one scale per (token, head) for K and for V: s = max|x| / Q (ASYM
  // values: s = (max - min) / L and the offset min, -0 made +0)
  for (int i = tid; i < 2 * kPage; i += kThreads) {
    const int which = i / kPage, r = i % kPage;
    if (r < lo || r >= hi || (!WITH_K && which == 0)) continue;
    const float* row = (which ? vtile : ktile) + r * LD;
    if constexpr (ASYM) {
      float mn = row[0], mx = row[0];
      for (int c = 1; c < D; ++c) {
        mn = fminf(mn, row[c]);
        mx = fmaxf(mx, row[c]);
      }
      mn = mn + 0.0f;
      const float s = (mx - mn) / kLevels;
      v_sc[r] = s;
      v_mn[r] = mn;
      reinterpret_cast<float*>(pg + p.off_vs)[r] = s;
      reinterpret_cast<float*>(pg + p.off_vz)[r] = mn;
    } else {
      float a = fabsf(row[0]);
      for (int c = 1; c < D; ++c) a = fmaxf(a, fabsf(row[c]));
      const float s = a / kQmax;
      (which ? v_sc : k_sc)[r] = s;
      reinterpret_cast<float*>(pg + (which ? p.off_vs : p.off_ks))[r] = s;
    }
  }
  __syncthreads();

  auto encode = [&](float x, float s) -> uint32_t { return quant_sym(x, s, kQmax, kMask); };
  // value code of token t, channel c
  auto encode_v = [&](int t, int c) -> uint32_t {
    if constexpr (ASYM) return quant_asym(vtile[t * LD + c], v_mn[t], v_sc[t], kLevels);
    else return encode(vtile[t * LD + c], v_sc[t]);
  };

  // K rows of the new tokens: whole words
  constexpr int ROW_WORDS = D * BITS / 32;
  uint32_t* kc = reinterpret_cast<uint32_t*>(pg + p.off_kc);
  if constexpr (BITS == 3) {
    // 3-bit fields straddle words: K rows in groups of 32 channels (3 words,
    // whole words of the token's row); V cols one column (32 tokens, 3
    // words) per thread, updating only the fields of tokens [lo, hi)
    constexpr int GPR = D / 32;
    for (int i = tid; i < (WITH_K ? (hi - lo) * GPR : 0); i += kThreads) {
      const int r = lo + i / GPR, gi = i % GPR;
      uint32_t wd[3] = {0u, 0u, 0u}, m[3] = {0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 32; ++j) put_field<3>(wd, m, j, encode(ktile[r * LD + 32 * gi + j], k_sc[r]));
      uint32_t* dst = kc + r * ROW_WORDS + 3 * gi;
      dst[0] = wd[0];
      dst[1] = wd[1];
      dst[2] = wd[2];
    }
    uint32_t* vc3 = reinterpret_cast<uint32_t*>(pg + p.off_vc);
    for (int c = tid; c < D; c += kThreads) {
      uint32_t wd[3] = {0u, 0u, 0u}, m[3] = {0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < kPage; ++t)
        if (t >= lo && t < hi) put_field<3>(wd, m, t, encode_v(t, c));
#pragma unroll
      for (int k = 0; k < 3; ++k) vc3[3 * c + k] = (vc3[3 * c + k] & ~m[k]) | wd[k];
    }
    return;
  }
  for (int i = tid; i < (WITH_K ? (hi - lo) * ROW_WORDS : 0); i += kThreads) {
    const int r = lo + i / ROW_WORDS;
    const int c0 = (i % ROW_WORDS) * FPW;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < FPW; ++j) word |= encode(ktile[r * LD + c0 + j], k_sc[r]) << (j * BITS);
    kc[r * ROW_WORDS + i % ROW_WORDS] = word;
  }
  // V cols: per channel, the words that hold fields of tokens [lo, hi)
  constexpr int COL_WORDS = kPage * BITS / 32;
  const int w_lo = lo / FPW, w_hi = (hi - 1) / FPW + 1;
  uint32_t* vc = reinterpret_cast<uint32_t*>(pg + p.off_vc);
  for (int i = tid; i < D * (w_hi - w_lo); i += kThreads) {
    const int c = i / (w_hi - w_lo);
    const int w = w_lo + i % (w_hi - w_lo);
    uint32_t word = 0, mask = 0;
#pragma unroll
    for (int j = 0; j < FPW; ++j) {
      const int t = w * FPW + j;
      if (t >= lo && t < hi) {
        word |= encode_v(t, c) << (j * BITS);
        mask |= kMask << (j * BITS);
      }
    }
    uint32_t* dst = vc + c * COL_WORDS + w;
    *dst = mask == 0xffffffffu ? word : ((*dst & ~mask) | word);
  }
}

// ---- FP8 (either format) and bfloat16 pages: byte-aligned codes ------------
// Every code is a whole byte (FP8) or a whole 16-bit word (bfloat16), so no
// token shares a word with another's field and no LDS staging or
// read-modify-write is needed: a thread takes a 4-token x 16-byte-chunk tile
// of the K rows and another of the V rows, issues its eight loads together,
// encodes, and stores K codes as row pieces and V codes as 4-token pieces of
// each channel's column. Lanes of the K tile run along a row (chunk fastest),
// lanes of the V tile along the tokens (token quad fastest), so both loads
// and stores touch whole 128-byte lines. FP8 quotients are the correctly
// rounded x / s, computed from the scale's reciprocal with two FMA
// corrections, and the codes come from the hardware conversion (clamped so
// it saturates). grid.x covers (pages of this launch) x (8 * CH tiles per
// page) flat, so that neighbouring blocks write neighbouring pages of one
// slab; grid y, z = KV head, sequence. Tokens outside [past, past + n) of a
// page are neither read nor written.
// FP8 values of the cache's open last page (fewer than 32 tokens) are kept in
// token rows, so that a token appended to it writes one contiguous row; a
// page is written as columns once it holds 32 tokens. The page that was open
// before the call and fills in it (the sequence's first page of the call) is
// the first 8 * CH tasks of block 0: that block copies the page's earlier
// value rows into LDS before any of its threads writes the page's columns.
// A block covers whole pages (256 threads, or one page of 8 * CH tasks when
// that is more).
// WITH_V false: the keys only (values in another cache type, written by
// another kernel)
template <int D, int IB>
constexpr int byte_append_threads() {
  return 8 * (D * IB / 16) > kThreads ? 8 * (D * IB / 16) : kThreads;
}

template <int SCHEME, int D, int IB, bool WITH_V = true>
__global__ __launch_bounds__((byte_append_threads<D, IB>())) void byte_append_kernel(AppendParams p,
                                                                                    int64_t pages) {
  constexpr int CB = SCHEME == KVQ_BF16_CACHE ? 2 : 1;   // bytes per code
  constexpr int CH = D * IB / 16;                          // 16-byte chunks per input row
  constexpr int EPC = 16 / IB;                             // elements per chunk
  constexpr int TPU = 8 * CH;                              // tiles per page
  constexpr int NTH = byte_append_threads<D, IB>();
  static_assert(NTH % TPU == 0, "a block covers whole pages");
  constexpr bool ROWS = CB == 1 && WITH_V;                 // FP8 values: open pages in rows
  const int64_t gtask = static_cast<int64_t>(blockIdx.x) * NTH + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  int64_t past, n;
  seq_counts(p, b, past, n);
  const int64_t end = past + n;
  const int64_t first = past / kPage;
  // the open page at the start of the call fills in it: its earlier value
  // rows become columns
  const bool closes = ROWS && past % kPage != 0 && end >= (first + 1) * kPage;
  __shared__ __attribute__((aligned(16))) uint8_t oldv[ROWS ? kPage * D : 16];
  if (closes && blockIdx.x == 0) {   // block-uniform
    const uint8_t* pv = p.pm.page(b, h, first) + p.off_vc;
    const int chunks = static_cast<int>(past % kPage) * D / 16;
    for (int i = threadIdx.x; i < chunks; i += NTH)
      *reinterpret_cast<uint4*>(oldv + 16 * i) = *reinterpret_cast<const uint4*>(pv + 16 * i);
    __syncthreads();   // read before any column of the page is written
  }
  // pages this sequence touches (at most `pages`, the launch's bound)
  const int64_t mine = n > 0 ? (end - 1) / kPage - first + 1 : 0;
  if (gtask >= (mine < pages ? mine : pages) * TPU) return;
  const int task = static_cast<int>(gtask % TPU);
  const int64_t page = first + gtask / TPU;
  const int lo = static_cast<int>((past > page * kPage ? past : page * kPage) - page * kPage);
  const int hi = static_cast<int>((end < page * kPage + kPage ? end : page * kPage + kPage) -
                                  page * kPage);
  uint8_t* pg = p.pm.page(b, h, page);
  constexpr int64_t ROW = static_cast<int64_t>(D) * IB;
  const int64_t row_stride = static_cast<int64_t>(p.kv_heads) * ROW;
  // input row of page token r (valid only for lo <= r < hi)
  const int64_t row0 = (static_cast<int64_t>(b) * p.stride + page * kPage - past) * row_stride +
                       static_cast<int64_t>(h) * ROW;

  const int kq = task / CH, kc = task % CH;   // K tile: tokens 4kq.., chunk kc
  const int vc = task / 8, vq = task % 8;     // V tile: chunk vc, tokens 4vq..
  uint4 kin[4], vin[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rk = 4 * kq + i, rv = 4 * vq + i;
    kin[i] = rk >= lo && rk < hi
                 ? *reinterpret_cast<const uint4*>(p.k_new + row0 + rk * row_stride + kc * 16)
                 : make_uint4(0, 0, 0, 0);
    vin[i] = WITH_V && rv >= lo && rv < hi
                 ? *reinterpret_cast<const uint4*>(p.v_new + row0 + rv * row_stride + vc * 16)
                 : make_uint4(0, 0, 0, 0);
  }

  auto widen = [](const uint4& v, float (&f)[EPC]) {
    if constexpr (IB == 2) {
      unpack_bf16x8(v, f);
    } else {
      f[0] = __uint_as_float(v.x);
      f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z);
      f[3] = __uint_as_float(v.w);
    }
  };
  // FP8: quotients by the per-head scale (correctly rounded from the
  // reciprocal, the IEEE division when it is out of range), then the hardware
  // conversion, two codes per instruction
  float ks = 1.0f, vs = 1.0f, kr = 1.0f, vr = 1.0f;
  bool exact = false;
  if constexpr (SCHEME != KVQ_BF16_CACHE) {
    ks = p.k_scale[h];
    vs = WITH_V ? p.v_scale[h] : 1.0f;
    kr = 1.0f / ks;
    vr = 1.0f / vs;
    exact = !(recip_usable(kr) && recip_usable(vr));
  }
  constexpr bool E5 = SCHEME == KVQ_FP8_E5M2;

  // K rows: EPC codes of one token row per store
  uint8_t* kdst = pg + p.off_kc + kc * EPC * CB;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * kq + i;
    if (r < lo || r >= hi) continue;
    float f[EPC];
    widen(kin[i], f);
    uint32_t w[EPC * CB / 4];
    if constexpr (CB == 1) {
      fp8_quotients(f, ks, kr, exact);
#pragma unroll
      for (int e = 0; e < EPC / 4; ++e)
        w[e] = fp8x2_encode<E5, true>(f[4 * e + 2], f[4 * e + 3],
                                      fp8x2_encode<E5, false>(f[4 * e], f[4 * e + 1], 0));
    } else {
#pragma unroll
      for (int e = 0; e < EPC / 2; ++e)
        w[e] = bf16_bits_rne(f[2 * e]) | (bf16_bits_rne(f[2 * e + 1]) << 16);
    }
    uint8_t* dst = kdst + static_cast<int64_t>(r) * D * CB;
    if constexpr (EPC * CB == 16) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (EPC * CB == 8) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    }
  }

  if constexpr (!WITH_V) return;
  // V cols: codes of tokens 4vq..4vq+3 of each of the chunk's channels
  float fv[4][EPC];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    widen(vin[i], fv[i]);
    if constexpr (CB == 1) fp8_quotients(fv[i], vs, vr, exact);
  }
  if constexpr (CB == 1) {
    if (hi < kPage) {
      // the page stays open: each token's EPC codes into its value row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * vq + i;
        if (r < lo || r >= hi) continue;
        uint32_t w[EPC / 4];
#pragma unroll
        for (int e = 0; e < EPC / 4; ++e)
          w[e] = fp8x2_encode<E5, true>(fv[i][4 * e + 2], fv[i][4 * e + 3],
                                        fp8x2_encode<E5, false>(fv[i][4 * e], fv[i][4 * e + 1], 0));
        uint8_t* dst = pg + p.off_vc + static_cast<int64_t>(r) * D + vc * EPC;
        if constexpr (EPC == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint32_t*>(dst) = w[0];
      }
      return;
    }
    // one dword of 4 token codes per channel; 4x4 transposes across the lane
    // quad that holds tokens 16m..16m+15 (vq = 4m + j, j = lane & 3) leave
    // lane j with channel 4t + j's 16 codes in dw[4t..4t+3], so the quad's
    // stores cover four whole 32-byte columns, 128 contiguous bytes
    uint32_t dw[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      dw[e] = fp8x2_encode<E5, true>(fv[2][e], fv[3][e], fp8x2_encode<E5, false>(fv[0][e], fv[1][e], 0));
    // the page filling in this call: its earlier tokens' codes from their rows
    const bool closing = closes && page == first;
    if (closing) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * vq + i;
        if (r >= lo) continue;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          dw[e] = (dw[e] & ~(0xFFu << (8 * i))) | (uint32_t(oldv[r * D + vc * EPC + e]) << (8 * i));
      }
    }
    const int lo_c = closing ? 0 : lo;   // first token whose column byte is written
    const int j = vq & 3, m = vq >> 2;
#pragma unroll
    for (int t = 0; t < EPC / 4; ++t) {
      uint32_t blk[4] = {dw[4 * t], dw[4 * t + 1], dw[4 * t + 2], dw[4 * t + 3]};
      quad_transpose(blk, j);
      uint8_t* dst = pg + p.off_vc + static_cast<int64_t>(vc * EPC + 4 * t + j) * kPage + 16 * m;
      if (16 * m >= lo_c && 16 * m + 16 <= hi) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(blk[0], blk[1], blk[2], blk[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 16 * m + i;
          if (r >= lo_c && r < hi) dst[i] = static_cast<uint8_t>(blk[i / 4] >> (8 * (i % 4)));
        }
      }
    }
  } else {
    const bool whole = 4 * vq >= lo && 4 * vq + 4 <= hi;
    uint8_t* vdst = pg + p.off_vc + static_cast<int64_t>(vc) * EPC * kPage * CB + 4 * vq * CB;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const uint32_t w0 = bf16_bits_rne(fv[0][e]) | (bf16_bits_rne(fv[1][e]) << 16);
      const uint32_t w1 = bf16_bits_rne(fv[2][e]) | (bf16_bits_rne(fv[3][e]) << 16);
      uint8_t* dst = vdst + e * kPage * CB;
      if (whole) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * vq + i;
          if (r >= lo && r < hi)
            reinterpret_cast<uint16_t*>(dst)[i] = static_cast<uint16_t>((i < 2 ? w0 : w1) >> (16 * (i & 1)));
        }
      }
    }
  }
}

// ---- dispatch ---------------------------------------------------------------

template <int D, int KB, int VB, int IB>
hipError_t run_kivi(const AppendArgs& a, const AppendParams& p, hipStream_t st) {
  const Geometry& g = a.g;
  int64_t flush_pages, ring_tokens;
  if (a.seq_past) {
    // ragged batch: bounds over every sequence (a sequence appending n tokens
    // flushes at most ceil(n / 32) pages and keeps at most min(n, R + 31) in
    // the ring); blocks past their own sequence's range return at once
    flush_pages = (a.n + kPage - 1) / kPage + 1;
    ring_tokens = a.n < g.residual + kPage ? a.n : g.residual + kPage;
  } else {
    const int64_t end = a.past + a.n;
    const int64_t q_old = kivi_quantised(a.past, g.residual);
    const int64_t q_new = kivi_quantised(end, g.residual);
    flush_pages = (q_new - q_old) / kPage;
    ring_tokens = end - (q_new > a.past ? q_new : a.past);
  }
  if (flush_pages > 0) {
    dim3 grid(static_cast<unsigned>(flush_pages), g.kv_heads, g.batch);
    if (g.outliers)
      hipLaunchKernelGGL((kivi_flush_kernel<D, KB, VB, IB, true>), grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((kivi_flush_kernel<D, KB, VB, IB, false>), grid, dim3(kThreads), 0, st, p);
  }
  if (ring_tokens > 0) {
    dim3 grid(static_cast<unsigned>(ring_tokens), g.kv_heads, g.batch);
    hipLaunchKernelGGL((ring_write_kernel<D, IB>), grid, dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

template <int SCHEME, int D, int BITS, int IB>
hipError_t run_token(const AppendArgs& a, const AppendParams& p, hipStream_t st) {
  const Geometry& g = a.g;
  // pages touched: exact for a uniform batch; for a ragged one the bound over
  // every sequence (n tokens touch at most ceil(n / 32) + 1 pages)
  const int64_t pages = a.seq_past ? (a.n + kPage - 1) / kPage + 1
                                   : (a.past + a.n - 1) / kPage - a.past / kPage + 1;
  if constexpr (SCHEME == KVQ_SYM_TOKEN) {
    dim3 grid(static_cast<unsigned>(pages), g.kv_heads, g.batch);
    hipLaunchKernelGGL((token_append_kernel<D, BITS, IB>), grid, dim3(kThreads), 0, st, p);
  } else {
    constexpr int64_t TPU = 8 * (D * IB / 16);
    constexpr int NTH = byte_append_threads<D, IB>();
    dim3 grid(static_cast<unsigned>((pages * TPU + NTH - 1) / NTH), g.kv_heads, g.batch);
    hipLaunchKernelGGL((byte_append_kernel<SCHEME, D, IB>), grid, dim3(NTH), 0, st, p, pages);
  }
  return hipGetLastError();
}

// Keys and values in different cache types: FP8 E4M3 key rows (the byte-code
// kernel, keys only), symmetric or KIVI (ASYM) value columns and their
// per-token scales (the per-token kernel, values only); the two write
// disjoint bytes of the pages.
template <int D, int IB, bool ASYM>
hipError_t run_fp8k_mixed(const AppendArgs& a, const AppendParams& p, hipStream_t st) {
  const Geometry& g = a.g;
  const int64_t pages = a.seq_past ? (a.n + kPage - 1) / kPage + 1
                                   : (a.past + a.n - 1) / kPage - a.past / kPage + 1;
  constexpr int64_t TPU = 8 * (D * IB / 16);
  constexpr int NTH = byte_append_threads<D, IB>();
  dim3 kgrid(static_cast<unsigned>((pages * TPU + NTH - 1) / NTH), g.kv_heads, g.batch);
  hipLaunchKernelGGL((byte_append_kernel<KVQ_FP8_E4M3, D, IB, false>), kgrid, dim3(NTH), 0, st, p, pages);
  dim3 vgrid(static_cast<unsigned>(pages), g.kv_heads, g.batch);
  switch (g.vbits) {
    case 2: hipLaunchKernelGGL((token_append_kernel<D, 2, IB, false, ASYM>), vgrid, dim3(kThreads), 0, st, p); break;
    case 3: hipLaunchKernelGGL((token_append_kernel<D, 3, IB, false, ASYM>), vgrid, dim3(kThreads), 0, st, p); break;
    case 4: hipLaunchKernelGGL((token_append_kernel<D, 4, IB, false, ASYM>), vgrid, dim3(kThreads), 0, st, p); break;
    default: hipLaunchKernelGGL((token_append_kernel<D, 8, IB, false, ASYM>), vgrid, dim3(kThreads), 0, st, p); break;
  }
  return hipGetLastError();
}

template <int D, int IB>
hipError_t dispatch_bits(const AppendArgs& a, const AppendParams& p, hipStream_t st) {
  const Geometry& g = a.g;
  if (g.scheme == KVQ_FP8K_SYMV) return run_fp8k_mixed<D, IB, false>(a, p, st);
  if (g.scheme == KVQ_FP8K_KIVIV) return run_fp8k_mixed<D, IB, true>(a, p, st);
  if (g.scheme == KVQ_FP8_E4M3) return run_token<KVQ_FP8_E4M3, D, 8, IB>(a, p, st);
  if (g.scheme == KVQ_FP8_E5M2) return run_token<KVQ_FP8_E5M2, D, 8, IB>(a, p, st);
  if (g.scheme == KVQ_BF16_CACHE) return run_token<KVQ_BF16_CACHE, D, 16, IB>(a, p, st);
  if (g.scheme == KVQ_SYM_TOKEN) {
    switch (g.bits) {
      case 2: return run_token<KVQ_SYM_TOKEN, D, 2, IB>(a, p, st);
      case 3: return run_token<KVQ_SYM_TOKEN, D, 3, IB>(a, p, st);
      case 4: return run_token<KVQ_SYM_TOKEN, D, 4, IB>(a, p, st);
      default: return run_token<KVQ_SYM_TOKEN, D, 8, IB>(a, p, st);
    }
  }
  switch (g.bits) {
    case 2: return run_kivi<D, 2, 2, IB>(a, p, st);
    case 3: return g.vbits == 2 ? run_kivi<D, 3, 2, IB>(a, p, st) : run_kivi<D, 3, 3, IB>(a, p, st);
    case 4:
      return g.vbits == 2 ? run_kivi<D, 4, 2, IB>(a, p, st)
             : g.vbits == 3 ? run_kivi<D, 4, 3, IB>(a, p, st) : run_kivi<D, 4, 4, IB>(a, p, st);
    default:
      return g.vbits == 2   ? run_kivi<D, 8, 2, IB>(a, p, st)
             : g.vbits == 3 ? run_kivi<D, 8, 3, IB>(a, p, st)
             : g.vbits == 4 ? run_kivi<D, 8, 4, IB>(a, p, st) : run_kivi<D, 8, 8, IB>(a, p, st);
  }
}

template <int D>
hipError_t dispatch_dtype(const AppendArgs& a, const AppendParams& p, hipStream_t st) {
  return a.g.in_bytes == 2 ? dispatch_bits<D, 2>(a, p, st) : dispatch_bits<D, 4>(a, p, st);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  AppendParams p{};
  p.pm = a.pm;
  p.layer_base = a.layer_base;
  p.k_new = static_cast<const uint8_t*>(a.k_new);
  p.v_new = static_cast<const uint8_t*>(a.v_new);
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  p.slab_bytes = g.slab_bytes;
  p.page_bytes = g.page_bytes;
  p.ring_base = g.pages_per_slab * g.page_bytes;
  p.past = a.past;
  p.n = a.n;
  p.stride = a.n;
  p.seq_past = a.seq_past;
  p.seq_new = a.seq_new;
  p.capacity = g.capacity;
  p.residual = g.residual;
  p.ring_slots = g.ring_slots > 0 ? g.ring_slots : 1;
  p.kv_heads = g.kv_heads;
  p.off_kc = g.off_kc;
  p.off_ks = g.off_ks;
  p.off_kz = g.off_kz;
  p.off_vc = g.off_vc;
  p.off_vs = g.off_vs;
  p.off_vz = g.off_vz;
  p.outliers = g.outliers;
  p.off_ko = g.off_ko;
  p.off_vo = g.off_vo;
  p.off_ki = g.off_ki;
  p.off_vi = g.off_vi;
  switch (g.d) {
    case 32: return dispatch_dtype<32>(a, p, st);
    case 64: return dispatch_dtype<64>(a, p, st);
    case 128: return dispatch_dtype<128>(a, p, st);
    default: return dispatch_dtype<256>(a, p, st);
  }
}

}  // namespace kvq
