// Device helpers shared by the gfx950 kernels of the W8A8 library.
//
// Build contract: compiled with -ffp-contract=off (no implicit FMA), IEEE
// fp32 division and square root, denormals preserved. Every fused
// multiply-add below is written out explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

constexpr int kWave = 64;
constexpr int kQmax = 127;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// BF16 <-> fp32
// ---------------------------------------------------------------------------

// Low / high BF16 of a packed dword, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Two fp32 -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  v2f f = {lo, hi};
  v2bf b = __builtin_convertvector(f, v2bf);
  return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

// Max over aligned groups of `width` lanes (width a power of two <= 64).
template <int kWidth>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
  for (int off = kWidth / 2; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// Quantisation of one value
//
// Definition: code = clamp(round_half_even(fl32(x / s)), -127, 127) with s the
// stored fp32 scale. For scales whose reciprocal is a normal fp32 number the
// quotient is formed without a divide: t = fl(x * r) with r = fl(1/s) is
// within an ulp of x/s, the residual e = fma(-t, s, x) is exact, and
// fma(e, r, t) is the correctly rounded quotient (Markstein's correction).
// Tiny scales take the IEEE division. Both routes are checked against the
// oracle over every (absmax, x) pair of BF16 values.
//
// The rounded quotient is turned into an integer by adding 1.5 * 2^23: for
// |t| < 2^22 the sum's low mantissa bits hold round_half_even(t) in two's
// complement, so its low byte is the INT8 code.
// ---------------------------------------------------------------------------

struct QuantParams {
  float s;       // stored scale (0 for an all-zero group)
  float r;       // fl32(1/s) when `fast`
  bool fast;
};

// Scales below this absmax threshold use the IEEE division path.
constexpr float kFastAbsmaxMin = 7.888609052210118e-31f;  // 2^-100

__device__ __forceinline__ QuantParams quant_params(float amax) {
  QuantParams p;
  p.s = amax / 127.0f;                 // one IEEE fp32 division
  p.fast = amax >= kFastAbsmaxMin;
  p.r = p.fast ? 1.0f / p.s : 0.0f;    // IEEE fp32 division
  return p;
}

// fl32(x / s): the reciprocal route (kFast, scale with a normal reciprocal)
// or the IEEE division (tiny or zero scales).
template <bool kFast>
__device__ __forceinline__ float quant_quotient(float x, const QuantParams& p) {
  if constexpr (kFast) {
    float t = x * p.r;
    float e = __builtin_fmaf(-t, p.s, x);
    return __builtin_fmaf(e, p.r, t);
  } else {
    return p.s == 0.0f ? 0.0f : x / p.s;
  }
}

// Low byte of the result is the INT8 code.
__device__ __forceinline__ uint32_t quant_code_bits(float t) {
  t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
  return __float_as_uint(t + 12582912.0f);   // 1.5 * 2^23
}

// Four codes (low bytes of four code words) packed into one dword.
__device__ __forceinline__ uint32_t pack_codes(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);  // [c0.b0, c1.b0, 0, 0]
  uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);  // [0, 0, c2.b0, c3.b0]
  return lo | hi;
}

// Absolute-value bits of a packed BF16 pair, max of the two halves as a
// 15-bit magnitude (order of non-negative BF16 patterns = order of values).
__device__ __forceinline__ uint32_t absmax_bits_bf16x2(uint32_t d, uint32_t m) {
  uint32_t lo = d & 0x7FFFu;
  uint32_t hi = (d >> 16) & 0x7FFFu;
  m = m > lo ? m : lo;
  return m > hi ? m : hi;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace w8a8
