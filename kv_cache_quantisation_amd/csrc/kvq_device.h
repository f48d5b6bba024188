// Device helpers shared by the kernels: dtype conversion, the exact
// quantisers, FP8 (E4M3FN, E5M2) conversion and wavefront reductions (wave64).
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

// Weight 2^(m - M) of a partial softmax state with running max m against the
// reference max M; 0 when M is -inf, i.e. when no token was seen at all (a
// wave, a block or a split without tokens, which a ragged batch can leave),
// where 2^(-inf - -inf) would be NaN.
__device__ __forceinline__ float exp2_rel(float m, float M) {
  return M == -INFINITY ? 0.0f : exp2f(m - M);
}

// Symmetric code: clamp(rint(x / s), -Q, Q), 0 when s == 0; returned as the
// low b bits of its two's complement.
__device__ __forceinline__ uint32_t quant_sym(float x, float s, float qmax, uint32_t mask) {
  if (s == 0.0f) return 0u;
  float r = rintf(x / s);
  r = fminf(fmaxf(r, -qmax), qmax);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & mask;
}

// fp32 -> bfloat16 bits, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ---- x / s correctly rounded from a reciprocal --------------------------------
// With r = RN(1/s), q0 = RN(x * r) is within 2 units in the last place of x / s.
// One correction q1 = RN(q0 + RN(x - s * q0) * r) (the residual by FMA)
// brings it within one unit, and a second gives RN(x / s) exactly: that is
// Markstein's theorem (radix 2, round to nearest: a reciprocal correctly
// rounded and a quotient within one unit make one such step correctly
// rounded). The steps need no overflow or underflow: callers use it only with
// 2^-60 <= |r| <= 2^60, and quotients outside [2^-100, 2^100) keep q0, whose
// FP8 code (a signed zero or the saturated maximum) is the same as that of
// RN(x / s).
__device__ __forceinline__ bool recip_usable(float r) {
  const float a = fabsf(r);
  return a >= 0x1p-60f && a <= 0x1p60f;
}

__device__ __forceinline__ float div_by_recip(float x, float s, float r) {
  const float q0 = x * r;
  float q = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
  q = __builtin_fmaf(__builtin_fmaf(-q, s, x), r, q);
  const float a = fabsf(q0);
  return a >= 0x1p-100f && a < 0x1p100f ? q : q0;
}

// x[i] <- RN(x[i] / s); exact (a reciprocal out of range) takes the division.
template <int N>
__device__ __forceinline__ void fp8_quotients(float (&x)[N], float s, float r, bool exact) {
  if (exact) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] / s;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = div_by_recip(x[i], s, r);
  }
}

// Two fp32 -> two FP8 codes in the low (HI false) or high (HI true) 16 bits of
// the result, the other half taken from old: the hardware conversion rounds to
// nearest with ties to even; clamping to the largest finite magnitude first
// makes it saturate (every value beyond it is nearest to it or would round
// past it), as the FP8 cache encoding does.
template <bool E5, bool HI>
__device__ __forceinline__ uint32_t fp8x2_encode(float a, float b, uint32_t old) {
  constexpr float FMAX = E5 ? 57344.0f : 448.0f;
  a = __builtin_amdgcn_fmed3f(a, -FMAX, FMAX);
  b = __builtin_amdgcn_fmed3f(b, -FMAX, FMAX);
  if constexpr (E5) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(a, b, static_cast<int>(old), HI));
  } else {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
  }
}

// Transposes a 4x4 dword matrix held one row per lane by the four lanes of a
// quad (j = lane & 3): afterwards lane j holds column j, a[i] = old row i of
// lane i. Two butterfly stages (partner lane j^2, then j^1) over DPP quad
// permutations; in each stage a lane keeps the entries whose column agrees
// with its own lane bit and swaps the others with its partner. Every lane of
// the quad must be active.
template <int K>
__device__ __forceinline__ void quad_transpose_stage(uint32_t (&a)[4], int j) {
  constexpr int kCtrl = K == 2 ? 0x4E : 0xB1;   // quad_perm [2,3,0,1] or [1,0,3,2]
  const bool hb = (j & K) != 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c & K) continue;
    const uint32_t send = hb ? a[c] : a[c ^ K];
    const uint32_t recv = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(send), kCtrl, 0xF, 0xF, false));
    a[c] = hb ? recv : a[c];
    a[c ^ K] = hb ? a[c ^ K] : recv;
  }
}

__device__ __forceinline__ void quad_transpose(uint32_t (&a)[4], int j) {
  quad_transpose_stage<2>(a, j);
  quad_transpose_stage<1>(a, j);
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
