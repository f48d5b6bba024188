// Wave-level helpers of the matrix-core decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- wave-level helpers ------------------------------------------------------

// HBM -> LDS copy of 16 bytes per active lane: lane l writes lds_base + 16 l.
// lds_base must be the same in every lane of the wave.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(base), "v"(src) : "memory");
}

// Waits until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt, lgkmcnt: no wait
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Waits until at most n (0..15; larger values wait for 15) vector-memory
// operations of this wave are outstanding.
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    default: wait_vm<15>(); break;
  }
}

// Waits for this wave's LDS operations.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// 2^x on the transcendental unit; results below 2^-126 flush to zero, which
// only drops negligible softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8 cat4h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, uint4{a, b, c, d});
}

template <typename V2>
__device__ __forceinline__ uint32_t bits32(V2 v) { return __builtin_bit_cast(uint32_t, v); }

// Byte SEL of y holds two 2-bit codes as FP4 E2M1 nibbles (code c reads as
// c / 2) -> the exact codes as f32 (low nibble first).
template <int SEL>
__device__ __forceinline__ float2 codes2_f32(uint32_t y) {
  const auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(y, 2.0f, SEL);
  return float2{r[0], r[1]};
}

// 16 two-bit codes (one word) -> two 8-channel fragments, channel order
// {0,2,1,3,4,6,5,7} within each 8.
__device__ __forceinline__ void codes2_frags(uint32_t w, half8& f0, half8& f1) {
  const uint32_t y0 = w & 0x33333333u, y1 = (w >> 2) & 0x33333333u;
  f0 = cat4h(bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 0)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 0)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 1)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 1)));
  f1 = cat4h(bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 2)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 2)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y0, 2.0f, 3)),
             bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(y1, 2.0f, 3)));
}

// 8 four-bit codes (one word) -> one fragment, channel order {0,2,1,3,4,6,5,7}.
__device__ __forceinline__ half8 codes4_frag(uint32_t w) {
  const uint32_t y0 = w & 0x0F0F0F0Fu, y1 = (w >> 4) & 0x0F0F0F0Fu;
  return cat4h(bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y0, 512.0f, false)),
               bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y1, 512.0f, false)),
               bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y0, 512.0f, true)),
               bits32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(y1, 512.0f, true)));
}

// Sum over aligned groups of 8 lanes (all lanes receive it).
// (The moves read a source lane for every lane, so an update with old value 0
// is the plain move; written that way the compiler folds each move into the
// add that consumes it.)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  return v;
}

// Sum over the 16 lanes of each DPP row (all lanes receive it).
__device__ __forceinline__ float row_sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);   // row_mirror
  return v;
}

// Value of lane l ^ 32.
__device__ __forceinline__ float xor32(float v) {
  const int lane = threadIdx.x & 63;
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                            false, false);
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// Value of lane l ^ 16 (within each half of the wave), by a swap of row
// pairs on the vector ALU: the swap hands each even row the odd row after it
// (second result) and each odd row the even row before it (first result). No
// LDS instruction, so a chain of these does not wait on LDS round trips.
__device__ __forceinline__ float xor16(float v) {
  const int lane = threadIdx.x & 63;
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                            false, false);
  return __builtin_bit_cast(float, ((lane >> 4) & 1) ? r[0] : r[1]);
}

// Maximum over the wave (all lanes receive it), by DPP moves and lane swaps
// (no LDS permutes).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, xor16(v));
  return fmaxf(v, xor32(v));
}

template <int SHIFT>
__device__ __forceinline__ float row_shl(float v) {  // lane l gets lane l+SHIFT of its row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x100 + SHIFT, 0xF, 0xF, false));
}

// Lane l gets v of lane l-SHIFT of its row; lanes with no such source keep `keep`.
template <int SHIFT>
__device__ __forceinline__ uint32_t shr_keep(uint32_t keep, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(keep), static_cast<int>(v),
                                                           0x110 + SHIFT, 0xF, 0xF, false));
}

// f32 pair -> packed f16 (hi) and packed f16 remainder (lo), hi + lo ~ x.
__device__ __forceinline__ void split_f16(float a, float b, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a, b);
  // a - hi as one mixed-precision fma per value, reading hi's f16 halves in
  // place (exact: hi is a truncation of a)
  const uint32_t hw = bits32(h);
  float ra, rb;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(hw), "v"(a));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(hw), "v"(b));
  const auto r = __builtin_amdgcn_cvt_pkrtz(ra, rb);
  hi = bits32(h);
  lo = bits32(r);
}

// f32 pair -> packed bf16 (hi, nearest) and packed bf16 remainder (lo); hi + lo
// carries 16 significant bits of each value at any magnitude (no subnormal
// floor, unlike f16), and the rounding is unbiased.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  // one conversion of the pair (left to itself the compiler converts a twice)
  uint32_t h;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(h) : "v"(a), "v"(b));
  const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xFFFF0000u);
  hi = h;
  lo = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(a - ha), static_cast<__bf16>(b - hb)});
}

// bf16 value of x by truncation (top 16 bits); x - trunc(x) is exact in f32.
__device__ __forceinline__ float bf16_trunc(float x) {
  return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
}
// Packs the bf16 top halves of a (low) and b (high) into one word.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Device-scope (all XCDs) relaxed store / load of a split partial.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Key rows of a page are copied HBM -> LDS with their 16-byte chunks permuted
// inside each row: logical chunk h of row r sits at chunk h ^ kswz<CPR>(r)
// (CPR = chunks per row, a power of two), so the rows that the 16 lanes of a
// wave read together fall into different LDS banks.
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (CPR >= 8) return r & 7;
  else return (r * CPR / 8) % CPR;
}

// LDS byte offset of byte b of key row r (rows of CPR chunks, permuted as above).
template <int CPR>
__device__ __forceinline__ int krow_off(int r, int b) {
  return r * (16 * CPR) + 16 * ((b >> 4) ^ kswz<CPR>(r)) + (b & 15);
}

}  // namespace kvq
