// Device helpers shared by the kernels: dtype conversion, the exact
// quantisers, FP8 E4M3FN conversion and wavefront reductions (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Converts 8 consecutive input elements held in 16 (bf16) or 32 (f32) bytes.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* o) {
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
  o[4] = __uint_as_float(v.z << 16);
  o[5] = __uint_as_float(v.z & 0xffff0000u);
  o[6] = __uint_as_float(v.w << 16);
  o[7] = __uint_as_float(v.w & 0xffff0000u);
}

// KIVI asymmetric code: clamp(rint((x - mn) / s), 0, L), 0 when s == 0.
// mn must already be canonical (+0 for a zero minimum). IEEE division.
__device__ __forceinline__ uint32_t quant_asym(float x, float mn, float s, float levels) {
  if (s == 0.0f) return 0u;
  float r = rintf((x - mn) / s);
  r = fminf(fmaxf(r, 0.0f), levels);
  return static_cast<uint32_t>(r);
}

// The same code as quant_asym, computed with a prepared reciprocal r of s
// (quant_rcp_prep): q = (x - mn) * r is within 2^-13 of the exactly rounded
// quotient for quotients up to 256 (v_rcp_f32 is within 1 ulp), so rint(q)
// equals rint of the IEEE quotient unless q is within 2^-12 of a
// half-integer; those rare elements take the IEEE division. r = 0 for s = 0
// gives code 0; r = NaN (s too small for the reciprocal) sends every element
// to the division.
__device__ __forceinline__ float quant_rcp_prep(float s) {
  return s == 0.0f ? 0.0f : (s >= 0x1p-100f ? __builtin_amdgcn_rcpf(s) : __builtin_nanf(""));
}
// (s is read only on the division path.)
__device__ __forceinline__ uint32_t quant_asym_rcp(float x, float mn, const float* s, float r,
                                                   float levels) {
  const float a = x - mn;
  const float ar = a * r;
  float q = rintf(ar);
  if (!(fabsf(ar - q) <= 0.5f - 0x1p-12f)) q = rintf(a / *s);
  return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(q, 0.0f, levels));
}

// Symmetric code: clamp(rint(x / s), -Q, Q), 0 when s == 0; returned as the
// low b bits of its two's complement.
__device__ __forceinline__ uint32_t quant_sym(float x, float s, float qmax, uint32_t mask) {
  if (s == 0.0f) return 0u;
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -qmax), qmax);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & mask;
}

// fp32 -> OCP E4M3FN, nearest with ties to even mantissa, saturating at 448,
// sign kept. Normal results round the fp32 significand to 3 bits with integer
// arithmetic; below 2^-6 the grid is uniform with step 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {
    mag = static_cast<uint32_t>(rintf(a * 512.0f));  // exact scaling, 0..8
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);                 // round to 3 mantissa bits, ties even
    mag = (b >> 20) - (120u << 3);                    // exponent bias 127 -> 7
  }
  return sign | mag;
}

// fp32 -> bfloat16 bits, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E5M2, nearest with ties to even mantissa, saturating at 57344
// (the largest finite value), sign kept. Normal results round the fp32
// significand to 2 bits; below 2^-14 the grid is uniform with step 2^-16.
__device__ __forceinline__ uint32_t e5m2_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (a >= 57344.0f) {
    mag = 0x7Bu;
  } else if (a < 6.103515625e-05f) {
    mag = static_cast<uint32_t>(rintf(a * 65536.0f));   // exact scaling, 0..4
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0xFFFFFu + ((b >> 21) & 1u);                 // round to 2 mantissa bits, ties even
    mag = (b >> 21) - (112u << 2);                    // exponent bias 127 -> 15
  }
  return sign | mag;
}

// OCP E5M2 byte -> fp32 (finite codes).
__device__ __forceinline__ float e5m2_decode(uint32_t c) {
  const uint32_t e = (c >> 2) & 0x1Fu;
  const uint32_t m = c & 3u;
  float v = e ? __uint_as_float(((e + 112u) << 23) | (m << 21))
              : static_cast<float>(m) * 1.52587890625e-05f;
  return (c & 0x80u) ? -v : v;
}

// OCP E4M3FN byte -> fp32 (finite codes).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
              : static_cast<float>(m) * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over the 32 lanes of each half of the wave.
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace kvq
