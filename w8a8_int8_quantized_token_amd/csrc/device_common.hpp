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
typedef unsigned v4u __attribute__((ext_vector_type(4)));
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

// fp32 -> the fp32 value of its BF16 rounding (nearest even), in one
// instruction: with a zero low half, the packed pair is that value's bits.
__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16x2(0.0f, v)); }

// GELU, erf form, of a BF16 value y: y/2 * erfc(-y / sqrt(2)) in fp32. erfc
// instead of 1 + erf keeps the digits of the small negative outputs.
__device__ __forceinline__ float gelu_erf(float y) {
  return 0.5f * y * erfcf(-y * 0.70710678118654752f);
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes)
// ---------------------------------------------------------------------------

// Within each 16-lane row, DPP moves (no LDS round trip): two quad swaps
// (lane ^ 1, lane ^ 2), then rotations of the row by 4 and 8 lanes. After
// the four steps every lane of a row holds an op over the whole row; the
// rows are then combined from lanes 0, 16, 32 and 48 with v_readlane.
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over each 16-lane row, in every lane of the row.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = umax(v, dpp_u32<kDppQuadXor1>(v));
  v = umax(v, dpp_u32<kDppQuadXor2>(v));
  v = umax(v, dpp_u32<kDppRowRor4>(v));
  return umax(v, dpp_u32<kDppRowRor8>(v));
}

// Max over the wave (uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max_u32(v);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return umax(umax(a, b), umax(c, d));
}

// Max over aligned groups of 16 lanes (one DPP row), in every lane.
template <int kWidth>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(kWidth == 16, "groups are DPP rows");
  return row_max_u32(v);
}

// Pairwise fp32 sum over the wave (uniform result): depth 4 within a row,
// then (row 0 + row 1) + (row 2 + row 3) from one lane of each row.
__device__ __forceinline__ float wave_sum_f32(float x) {
  uint32_t v = __float_as_uint(x);
  v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<kDppQuadXor1>(v)));
  v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<kDppQuadXor2>(v)));
  v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<kDppRowRor4>(v)));
  v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<kDppRowRor8>(v)));
  const float a = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 0));
  const float b = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const float c = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 32));
  const float d = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return (a + b) + (c + d);
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

// Low byte of the result is the INT8 code. On the reciprocal route no clamp
// is needed: |x| <= absmax and s = fl32(absmax / 127) >= absmax / 127 /
// (1 + 2^-24), so |x / s| <= 127 (1 + 2^-24) and its correct rounding is at
// most 127 + 2^-17 < 127.5 for every finite x: the code is at most 127 in
// magnitude. The division route (scales that may be subnormal, with a
// relative error up to about 2^-9) keeps the clamp, one v_med3_f32.
template <bool kFast>
__device__ __forceinline__ uint32_t quant_code_bits(float t) {
  if constexpr (!kFast) t = __builtin_amdgcn_fmed3f(t, -127.0f, 127.0f);
  return __float_as_uint(t + 12582912.0f);   // 1.5 * 2^23
}

// The codes of four quotients (clamped as quant_code_bits does) in one
// dword. Each magic-number add is an SDWA form that writes only the low byte
// of its sum, into byte k of the result (the other bytes kept), so the bytes
// need no separate packing.
template <bool kFast>
__device__ __forceinline__ uint32_t code_bytes4(float t0, float t1, float t2, float t3) {
  if constexpr (!kFast) {
    t0 = __builtin_amdgcn_fmed3f(t0, -127.0f, 127.0f);
    t1 = __builtin_amdgcn_fmed3f(t1, -127.0f, 127.0f);
    t2 = __builtin_amdgcn_fmed3f(t2, -127.0f, 127.0f);
    t3 = __builtin_amdgcn_fmed3f(t3, -127.0f, 127.0f);
  }
  const float magic = 12582912.0f;   // 1.5 * 2^23
  uint32_t d;
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD "
      "src1_sel:DWORD"
      : "=v"(d) : "v"(t0), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD"
      : "+v"(d) : "v"(t1), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD"
      : "+v"(d) : "v"(t2), "s"(magic));
  asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
      "src1_sel:DWORD"
      : "+v"(d) : "v"(t3), "s"(magic));
  return d;
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
