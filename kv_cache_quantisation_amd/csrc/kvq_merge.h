// Merge of the split-softmax partials of a (sequence, KV head) across blocks,
// shared by the decode kernels.
//
// Each block of a (sequence, KV head) counts its arrival first, then combines
// its waves while the count is in flight. The block that arrives last keeps
// its own state in registers and merges the partials the other blocks store;
// every other block stores its partial and ends. A stored element holds the
// complement of the float's bits, so a slot that reads zero has not been
// written yet in this call: the last block polls such slots (the blocks that
// write them have already arrived, so they are running and the wait ends).
// No float produced by arithmetic has all 32 bits set (the quiet NaN of the
// hardware is positive), so no written value reads as zero. The merging block
// returns every slot it read, and the arrival counter, to zero, so a
// workspace is all zero between calls.
//
// Softmax merge (log2 domain): M = max_s m_s, out = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"

namespace kvq {

__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), ~__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t peek_partial(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void clear_partial(float* p) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls of one slot before giving up (about 0.2 s): a slot still empty then
// reads as NaN, so the output shows it instead of the kernel hanging.
constexpr int kPollLimit = 1 << 21;

// Re-reads *x from p until it is non-zero (bounded).
__device__ __forceinline__ void poll_until_written(const float* p, uint32_t& x) {
  for (int n = 0; x == 0u && n < kPollLimit; ++n) {
    __builtin_amdgcn_s_sleep(2);
    x = peek_partial(p);
  }
}

// Arrival of one block at its (sequence, KV head): the count before it.
__device__ __forceinline__ int count_arrival(int* counter) {
  return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A non-merging block stores its combined state: elements i = tid + e*NTH
// (head i / D, channel i % D) of its row. part_rh: the row's partials for
// this KV head's first query head, [HG][splits][D + 2] (m, l, o[D]).
template <int D, int HG, int NTH>
__device__ __forceinline__ void store_partial(float* part_rh, int splits, int split, const float* own_m,
                                              const float* own_l, const float* own_o, int tid) {
  constexpr int PER = (HG * D + NTH - 1) / NTH;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = tid + e * NTH;
    if (i < HG * D) {
      const int hh = i / D, c = i % D;
      float* part = part_rh + (static_cast<int64_t>(hh) * splits + split) * (D + 2);
      put_partial(part + 2 + c, own_o[e]);
      if (c == 0) {
        put_partial(part, own_m[e]);
        put_partial(part + 1, own_l[e]);
      }
    }
  }
}

// The last block merges every (query row, split) of sequence b, KV head h
// and writes the outputs out[r][h*HG + hh][c]; its own state (row `row`,
// split `split`) comes from registers (row -1: none; every slot is read).
// Then it clears what it read and the counter. partials: [rows][q_heads][splits][D + 2].
template <int D, int HG, int NTH>
__device__ __forceinline__ void merge_partials(float* partials, float* out, int* counter, int q_heads,
                                               int splits, int nq, int b, int h, int row, int split,
                                               const float* own_m, const float* own_l, const float* own_o,
                                               int tid) {
  constexpr int PER = (HG * D + NTH - 1) / NTH;
  for (int r = b * nq; r < (b + 1) * nq; ++r) {
    float* part_rh = partials + (static_cast<int64_t>(r) * q_heads + h * HG) * splits * (D + 2);
    const bool mine_row = r == row;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * NTH;
      if (i < HG * D) {
        const int hh = i / D, c = i % D;
        const float* part = part_rh + static_cast<int64_t>(hh) * splits * (D + 2);
        float M = -INFINITY, so = 0.f, sl = 0.f;
        for (int s0 = 0; s0 < splits; s0 += 8) {
          // the loads of 8 splits are issued together, then checked
          uint32_t xm[8], xl[8], xo[8];
          bool use[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int s = s0 + k;
            use[k] = s < splits && !(mine_row && s == split);
            const float* ps = part + (use[k] ? s : 0) * (D + 2);
            xm[k] = use[k] ? peek_partial(ps) : 1u;
            xl[k] = use[k] ? peek_partial(ps + 1) : 1u;
            xo[k] = use[k] ? peek_partial(ps + 2 + c) : 1u;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (use[k] && (xm[k] == 0u || xl[k] == 0u || xo[k] == 0u)) {   // not written yet
              const float* ps = part + (s0 + k) * (D + 2);
              poll_until_written(ps, xm[k]);
              poll_until_written(ps + 1, xl[k]);
              poll_until_written(ps + 2 + c, xo[k]);
            }
          }
          float mv[8], lv[8], ov[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const bool own = mine_row && s0 + k == split;
            mv[k] = use[k] ? __uint_as_float(~xm[k]) : (own ? own_m[e] : -INFINITY);
            lv[k] = use[k] ? __uint_as_float(~xl[k]) : (own ? own_l[e] : 0.f);
            ov[k] = use[k] ? __uint_as_float(~xo[k]) : (own ? own_o[e] : 0.f);
          }
          float bm = -INFINITY;
#pragma unroll
          for (int k = 0; k < 8; ++k) bm = fmaxf(bm, mv[k]);
          const float Mn = fmaxf(M, bm);
          const float a = exp2_rel(M, Mn);
          so *= a;
          sl *= a;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float w = exp2_rel(mv[k], Mn);   // absent split: m = -inf, weight 0
            sl = fmaf(w, lv[k], sl);
            so = fmaf(w, ov[k], so);
          }
          M = Mn;
        }
        out[(static_cast<int64_t>(r) * q_heads + h * HG + hh) * D + c] = so / sl;
      }
    }
  }
  // every thread has read m and l of its heads before they are cleared
  __syncthreads();
  for (int r = b * nq; r < (b + 1) * nq; ++r) {
    float* part_rh = partials + (static_cast<int64_t>(r) * q_heads + h * HG) * splits * (D + 2);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = tid + e * NTH;
      if (i < HG * D) {
        const int hh = i / D, c = i % D;
        float* part = part_rh + static_cast<int64_t>(hh) * splits * (D + 2);
        for (int s = 0; s < splits; ++s) {
          if (r == row && s == split) continue;   // never stored
          float* ps = part + s * (D + 2);
          clear_partial(ps + 2 + c);
          if (c == 0) {
            clear_partial(ps);
            clear_partial(ps + 1);
          }
        }
      }
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace kvq
