// Activation / weight quantisation kernels for gfx950.
//
// Per-token dynamic INT8 quantisation ("TurboDiffusion Integration Notes",
// section "Reused Components", W8A8 Linear bullet) and its RMSNorm-fused form
// (same section, FastNorm bullet). The path is HBM-bound: each row is read
// once as BF16 and written once as INT8.
//
// Layout of the work: one 64-lane wave owns one row. Lane l holds 16-byte
// vectors l, l+64, l+128, ... of the row (eight BF16 each), so every load
// instruction of a wave reads 1 KiB of contiguous row data. The whole row
// stays in registers between the absmax reduction and the quantisation, so
// HBM sees it exactly once. Rows longer than the register budget fall back to
// a two-pass loop that re-reads the row (from L2).
#include <atomic>

#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

constexpr int kRowsPerBlock = 4;   // 4 waves of 64 lanes, one row each
constexpr int kMaxSplitWaves = 16; // waves per row of the few-rows kernel

struct alignas(16) U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 load_nt(const U4* p) {
  U4 v;
  v.x = __builtin_nontemporal_load(&p->x);
  v.y = __builtin_nontemporal_load(&p->y);
  v.z = __builtin_nontemporal_load(&p->z);
  v.w = __builtin_nontemporal_load(&p->w);
  return v;
}

// Absolute maxima kept as two 16-bit lanes (low and high BF16 of each pair):
// the magnitude bits of non-negative BF16 order like the values, so a packed
// unsigned 16-bit max (v_pk_max_u16) takes two maxima per instruction.
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax2_u4(const U4& v, uint32_t m2) {
  const v2u16 a = __builtin_bit_cast(v2u16, v.x & 0x7FFF7FFFu);
  const v2u16 b = __builtin_bit_cast(v2u16, v.y & 0x7FFF7FFFu);
  const v2u16 c = __builtin_bit_cast(v2u16, v.z & 0x7FFF7FFFu);
  const v2u16 d = __builtin_bit_cast(v2u16, v.w & 0x7FFF7FFFu);
  const v2u16 t = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(t, __builtin_bit_cast(v2u16, m2)));
}
__device__ __forceinline__ uint32_t fold_absmax(uint32_t m2) {
  const uint32_t lo = m2 & 0xFFFFu, hi = m2 >> 16;
  return lo > hi ? lo : hi;
}
__device__ __forceinline__ uint32_t absmax_u4(const U4& v, uint32_t m) {
  const uint32_t r = fold_absmax(absmax2_u4(v, 0u));
  return r > m ? r : m;
}

// Eight BF16 -> eight INT8 codes (two dwords).
template <bool kFast>
__device__ __forceinline__ uint2 quant_u4(const U4& v, const QuantParams& p) {
  uint32_t c[8];
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = quant_code_bits<kFast>(quant_quotient<kFast>(bf16_lo(d[i]), p));
    c[2 * i + 1] = quant_code_bits<kFast>(quant_quotient<kFast>(bf16_hi(d[i]), p));
  }
  return make_uint2(pack_codes(c[0], c[1], c[2], c[3]), pack_codes(c[4], c[5], c[6], c[7]));
}

__device__ __forceinline__ uint2 quant_u4(const U4& v, const QuantParams& p) {
  return p.fast ? quant_u4<true>(v, p) : quant_u4<false>(v, p);
}

// Lane `lane` holds vectors lane + 64 j of the row (kFull: all of them exist).
template <int kVpl, bool kFull>
__device__ __forceinline__ bool has_vec(int lane, int j, int nvec) {
  return kFull || lane + j * kWave < nvec;
}

// Quantise a register-resident row with one scale; the fast/slow choice is
// uniform over the row, so it is taken once.
template <int kVpl, bool kFull, bool kFast>
__device__ __forceinline__ void store_row_codes(const U4 (&v)[kVpl], uint2* qr, int lane, int nvec,
                                                const QuantParams& p) {
#pragma unroll
  for (int j = 0; j < kVpl; ++j)
    if (has_vec<kVpl, kFull>(lane, j, nvec)) qr[lane + j * kWave] = quant_u4<kFast>(v[j], p);
}

// Unpredicated loads: a lane past the end of a short row re-reads the row's
// last vector (always in bounds, nvec >= 1) and then zeroes it, so the loads
// issue back to back with no branches around them.
// kStream: data read once (non-temporal hint); otherwise a cached load.
template <int kVpl, bool kFull, bool kStream = true>
__device__ __forceinline__ void load_row(U4 (&v)[kVpl], const U4* xr, int lane, int nvec) {
#pragma unroll
  for (int j = 0; j < kVpl; ++j) {
    const int idx = lane + j * kWave;
    const U4* src = xr + (kFull || idx < nvec ? idx : nvec - 1);
    if constexpr (kFull) {
      v[j] = kStream ? load_nt(src) : *src;
    } else {
      const U4 t = kStream ? load_nt(src) : *src;
      const bool in = idx < nvec;
      v[j] = U4{in ? t.x : 0u, in ? t.y : 0u, in ? t.z : 0u, in ? t.w : 0u};
    }
  }
}

// ---------------------------------------------------------------------------
// Per-row (group (1, cols)) and per-128-block (group (1, 128)) quantisation,
// row held in registers: kVpl 16-byte vectors per lane. kFull: the row is
// exactly kVpl * 64 vectors long, so no lane needs a bounds check.
// ---------------------------------------------------------------------------
template <int kVpl, bool kGroup128, bool kFull>
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                       int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;                       // whole wave leaves together
  const int nvec = (int)(cols >> 3);
  const U4* xr = reinterpret_cast<const U4*>(x + row * ldx);
  U4 v[kVpl];
  load_row<kVpl, kFull>(v, xr, lane, nvec);
  uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
  if constexpr (!kGroup128) {
    uint32_t m2 = 0;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) m2 = absmax2_u4(v[j], m2);
    const uint32_t m = wave_max_u32(fold_absmax(m2));
    const QuantParams p = quant_params(bf16_bits_to_float(m));
    if (p.fast) store_row_codes<kVpl, kFull, true>(v, qr, lane, nvec, p);
    else store_row_codes<kVpl, kFull, false>(v, qr, lane, nvec, p);
    if (lane == 0) scale[row] = p.s;
  } else {
    // vector idx covers columns [8 idx, 8 idx + 8); 16 consecutive vectors
    // (16 lanes) form one 128-wide group.
    const int64_t ngroups = cols >> 7;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) {
      const int idx = lane + j * kWave;
      uint32_t m = group_max_u32<16>(absmax_u4(v[j], 0u));
      const QuantParams p = quant_params(bf16_bits_to_float(m));
      if (has_vec<kVpl, kFull>(lane, j, nvec)) {
        qr[idx] = quant_u4(v[j], p);
        if ((lane & 15) == 0) scale[row * ngroups + (idx >> 4)] = p.s;
      }
    }
  }
}

// Few rows (fewer than the chip holds waves): one workgroup of S waves per
// row, S = blockDim.x / 64. Wave w holds vectors lane + 64 (w + S j), j <
// kVpl, so each load still reads 1 KiB of contiguous row data; the row's
// absmax is the maximum of the S wave maxima, exchanged through LDS. The
// arithmetic is the per-row kernel's, so codes and scales are identical.
// (1, 128) groups are 16 consecutive vectors, which stay in one wave.
template <int kVpl, bool kGroup128, bool kFull>
__global__ __launch_bounds__(kMaxSplitWaves * kWave)
void quant_rows_split_kernel(const uint16_t* __restrict__ x, int64_t cols, int64_t ldx,
                             int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale) {
  __shared__ uint32_t wave_max[kMaxSplitWaves];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int64_t row = blockIdx.x;
  const int nvec = (int)(cols >> 3);
  const U4* xr = reinterpret_cast<const U4*>(x + row * ldx);
  uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
  U4 v[kVpl];
#pragma unroll
  for (int j = 0; j < kVpl; ++j) {
    const int idx = lane + kWave * (w + S * j);
    const U4 t = load_nt(xr + (kFull || idx < nvec ? idx : nvec - 1));
    const bool in = kFull || idx < nvec;
    v[j] = U4{in ? t.x : 0u, in ? t.y : 0u, in ? t.z : 0u, in ? t.w : 0u};
  }
  if constexpr (!kGroup128) {
    uint32_t m2 = 0;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) m2 = absmax2_u4(v[j], m2);
    const uint32_t mw = wave_max_u32(fold_absmax(m2));
    if (lane == 0) wave_max[w] = mw;
    __syncthreads();
    uint32_t m = 0;
    for (int i = 0; i < S; ++i) m = umax(m, wave_max[i]);
    const QuantParams p = quant_params(bf16_bits_to_float(m));
#pragma unroll
    for (int j = 0; j < kVpl; ++j) {
      const int idx = lane + kWave * (w + S * j);
      if (kFull || idx < nvec) qr[idx] = quant_u4(v[j], p);
    }
    if (threadIdx.x == 0) scale[row] = p.s;
  } else {
    const int64_t ngroups = cols >> 7;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) {
      const int idx = lane + kWave * (w + S * j);
      const uint32_t m = group_max_u32<16>(absmax_u4(v[j], 0u));
      const QuantParams p = quant_params(bf16_bits_to_float(m));
      if (kFull || idx < nvec) {
        qr[idx] = quant_u4(v[j], p);
        if ((lane & 15) == 0) scale[row * ngroups + (idx >> 4)] = p.s;
      }
    }
  }
}

// Rows too long for the register-resident kernel: two passes over the row.
template <bool kGroup128>
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void quant_rows_long_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                            int64_t ldx, int8_t* __restrict__ q, int64_t ldq,
                            float* __restrict__ scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t nvec = cols >> 3;
  const U4* xr = reinterpret_cast<const U4*>(x + row * ldx);
  uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
  if constexpr (!kGroup128) {
    uint32_t m = 0;
    for (int64_t idx = lane; idx < nvec; idx += kWave) m = absmax_u4(xr[idx], m);
    m = wave_max_u32(m);
    const QuantParams p = quant_params(bf16_bits_to_float(m));
    for (int64_t idx = lane; idx < nvec; idx += kWave) qr[idx] = quant_u4(xr[idx], p);
    if (lane == 0) scale[row] = p.s;
  } else {
    const int64_t ngroups = cols >> 7;
    for (int64_t base = 0; base < nvec; base += kWave) {
      const int64_t idx = base + lane;
      const U4 v = idx < nvec ? xr[idx] : U4{0, 0, 0, 0};
      uint32_t m = group_max_u32<16>(absmax_u4(v, 0u));
      const QuantParams p = quant_params(bf16_bits_to_float(m));
      if (idx < nvec) {
        qr[idx] = quant_u4(v, p);
        if ((lane & 15) == 0) scale[row * ngroups + (idx >> 4)] = p.s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// (128, 128) groups: one workgroup of 256 threads per block of 128 rows x 128
// columns (the last row group may be shorter). Used once per weight, when the
// model is initialised.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void quant_block128_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                           int64_t ldx, int8_t* __restrict__ q, int64_t ldq,
                           float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int64_t gr = blockIdx.y, gc = blockIdx.x;
  const int64_t r0 = gr * 128;
  const int64_t nr = rows - r0 < 128 ? rows - r0 : 128;
  // 128 rows x 16 vectors = 2048 vectors, 8 per thread
  const int t = threadIdx.x;
  U4 v[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = t + i * 256;
    const int r = e >> 4, c = e & 15;
    if (r < nr) {
      v[i] = reinterpret_cast<const U4*>(x + (r0 + r) * ldx + gc * 128)[c];
      m = absmax_u4(v[i], m);
    } else {
      v[i] = U4{0, 0, 0, 0};
    }
  }
  m = wave_max_u32(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < 4; ++w) m = m > red[w] ? m : red[w];
  const QuantParams p = quant_params(bf16_bits_to_float(m));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = t + i * 256;
    const int r = e >> 4, c = e & 15;
    if (r < nr) reinterpret_cast<uint2*>(q + (r0 + r) * ldq + gc * 128)[c] = quant_u4(v[i], p);
  }
  if (t == 0) scale[gr * (cols >> 7) + gc] = p.s;
}

// ---------------------------------------------------------------------------
// RMSNorm + per-token quantisation, row in registers.
//   r = fl32(1 / sqrt(sum(x^2) / K + eps)), the sum of exact squares in fp64;
//   y = bf16(fl32(fl32(x * r) * gamma)); codes and scale from y.
// ---------------------------------------------------------------------------
// Sum of the eight exact squares of a vector in fp32: each v_dot2 adds two
// BF16 squares (exact products), then a pairwise tree.
__device__ __forceinline__ float sumsq8_f32(const U4& v) {
  const auto bf = [](uint32_t d) { return __builtin_bit_cast(v2bf, d); };
  const float a = __builtin_amdgcn_fdot2_f32_bf16(bf(v.x), bf(v.x), 0.0f, false);
  const float b = __builtin_amdgcn_fdot2_f32_bf16(bf(v.y), bf(v.y), 0.0f, false);
  const float c = __builtin_amdgcn_fdot2_f32_bf16(bf(v.z), bf(v.z), 0.0f, false);
  const float d = __builtin_amdgcn_fdot2_f32_bf16(bf(v.w), bf(v.w), 0.0f, false);
  return (a + b) + (c + d);
}

// Pairwise sum of t[lo, hi).
template <int kLo, int kHi>
__device__ __forceinline__ float tree_sum(const float* t) {
  if constexpr (kHi - kLo == 1) {
    return t[kLo];
  } else {
    constexpr int kMid = kLo + (kHi - kLo) / 2;
    return tree_sum<kLo, kMid>(t) + tree_sum<kMid, kHi>(t);
  }
}

// fp64 sum of exact squares, for rows whose fp32 sum leaves the safe range.
// The words pass through an empty asm so the compiler cannot share their
// BF16 -> fp32 unpacking with the normalisation that follows: sharing hoists
// the unpacking above this rarely taken branch and keeps 64 unpacked floats
// live for the whole row.
__device__ __forceinline__ double sumsq_u4(const U4& v, double acc) {
  uint32_t d[4] = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = (double)bf16_lo(d[i]);
    const double b = (double)bf16_hi(d[i]);
    acc = __builtin_fma(a, a, acc);
    acc = __builtin_fma(b, b, acc);
  }
  return acc;
}

// y = bf16(fl32(fl32(x * r) * g)) for eight elements, repacked as BF16 pairs.
__device__ __forceinline__ U4 rmsnorm_u4(const U4& v, const U4& g, float r) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  const uint32_t e[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = (bf16_lo(d[i]) * r) * bf16_lo(e[i]);
    const float hi = (bf16_hi(d[i]) * r) * bf16_hi(e[i]);
    o[i] = pack_bf16x2(lo, hi);
  }
  return U4{o[0], o[1], o[2], o[3]};
}

// One row: r from the sum of squares, y = bf16(x r g) in place, absmax,
// codes and the row's scale (and r) written out.
template <int kVpl, bool kFull, int kChunk>
__device__ __forceinline__ void rmsnorm_quant_row(U4 (&v)[kVpl], const U4* g, const U4* gr,
                                                  int lane, int nvec, int64_t cols, float eps,
                                                  uint2* qr, float* scale_out,
                                                  float* inv_rms_out) {
  // Sum of squares in fp32, pairwise from the squares up (depth about
  // log2(cols) + 2, all terms non-negative): relative error at most about
  // (log2(cols) + 4) * 2^-24, so r is within half that plus one rounding of
  // the fp64 reference. Rows whose fp32 sum is huge (squares may overflow)
  // or tiny (squares may be subnormal) take an fp64 sum instead; the choice
  // is uniform over the wave.
  float part[kVpl];
#pragma unroll
  for (int j = 0; j < kVpl; ++j) part[j] = sumsq8_f32(v[j]);
  const float ss32 = wave_sum_f32(tree_sum<0, kVpl>(part));
  double ss;
  if (ss32 >= 0x1p-80f && ss32 <= 0x1p100f) {
    ss = (double)ss32;
  } else {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) acc = sumsq_u4(v[j], acc);
    ss = wave_sum_f64(acc);
  }
  const double r64 = 1.0 / __builtin_sqrt(ss / (double)cols + (double)eps);
  const float r = (float)r64;
  // Gains: g holds all kVpl vectors (kChunk == kVpl), or null and they are
  // fetched from gr in chunks of kChunk.
  uint32_t m2 = 0;
#pragma unroll
  for (int j0 = 0; j0 < kVpl; j0 += kChunk) {
    U4 gc[kChunk];
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) {
      const int j = j0 + jj;
      if (j < kVpl) {
        if constexpr (kChunk == kVpl) {
          // through an empty asm: in a loop over rows the compiler would
          // otherwise hoist the unpacking of these loop-invariant words and
          // hold 64 unpacked floats instead of 32 packed ones
          U4 t = g[j];
          asm volatile("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
          gc[jj] = t;
        } else {
          const int idx = lane + j * kWave;
          gc[jj] = gr[kFull || idx < nvec ? idx : nvec - 1];
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < kChunk && j0 + jj < kVpl; ++jj) {
      const int j = j0 + jj;
      v[j] = rmsnorm_u4(v[j], gc[jj], r);   // padding: x = 0 gives y = 0
      m2 = absmax2_u4(v[j], m2);
    }
  }
  const uint32_t m = wave_max_u32(fold_absmax(m2));
  const QuantParams p = quant_params(bf16_bits_to_float(m));
  if (p.fast) store_row_codes<kVpl, kFull, true>(v, qr, lane, nvec, p);
  else store_row_codes<kVpl, kFull, false>(v, qr, lane, nvec, p);
  if (lane == 0) {
    *scale_out = p.s;
    if (inv_rms_out) *inv_rms_out = r;
  }
}

// One wave per row. Short rows load the gains up front; long rows (over 16
// vectors per lane) fetch them in chunks after the reduction to stay within
// the register budget.
template <int kVpl, bool kFull>
__global__ __launch_bounds__(kRowsPerBlock * kWave)
void rmsnorm_quant_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                          float eps, int64_t rows, int64_t cols, int64_t ldx,
                          int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale,
                          float* __restrict__ inv_rms) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nvec = (int)(cols >> 3);
  const U4* gr = reinterpret_cast<const U4*>(gamma);
  constexpr bool kGainsEarly = kVpl <= 16;
  U4 v[kVpl];
  U4 g[kGainsEarly ? kVpl : 1];
  load_row<kVpl, kFull>(v, reinterpret_cast<const U4*>(x + row * ldx), lane, nvec);
  if constexpr (kGainsEarly) load_row<kVpl, kFull, false>(g, gr, lane, nvec);
  rmsnorm_quant_row<kVpl, kFull, kGainsEarly ? kVpl : 8>(
      v, g, gr, lane, nvec, cols, eps, reinterpret_cast<uint2*>(q + row * ldq), scale + row,
      inv_rms ? inv_rms + row : nullptr);
}

// ---------------------------------------------------------------------------
// LayerNorm + adaLN modulation + per-token quantisation, row in registers.
//   mu = mean(x), r = fl32(1 / sqrt(mean((x - mu)^2) + eps)), the two sums in
//   fp32 pairwise (fp64 for rows outside the safe range);
//   y = bf16(fl32(fl32(fl32(fl32(x - mu) * r) * gamma) + beta));
//   z = bf16(fl32(bf16(fl32(y * m)) + shift)), m = bf16(fl32(1 + scale));
//   codes and scale from z. gamma, beta, scale and shift are optional
//   (a null pointer leaves the step out).
// ---------------------------------------------------------------------------
constexpr uint32_t kBf16OnePair = 0x3F803F80u;   // BF16 (1.0, 1.0)

// Sum of the eight elements: each v_dot2 adds a BF16 pair (times 1) to its
// accumulator; two chains of two, then one add (depth 3). The first dot of a
// chain is written out so that its zero accumulator is the inline constant
// (the compiler's form zeroes a register first).
__device__ __forceinline__ float dot2_bf16_ones(uint32_t w) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(w), "s"(kBf16OnePair));
  return r;
}
__device__ __forceinline__ float sum8_f32(const U4& v) {
  const auto bf = [](uint32_t d) { return __builtin_bit_cast(v2bf, d); };
  const v2bf one = bf(kBf16OnePair);
  const float a = __builtin_amdgcn_fdot2_f32_bf16(bf(v.y), one, dot2_bf16_ones(v.x), false);
  const float b = __builtin_amdgcn_fdot2_f32_bf16(bf(v.w), one, dot2_bf16_ones(v.z), false);
  return a + b;
}

// Sum of the eight squared deviations from mu, pairwise.
__device__ __forceinline__ float sqdev8_f32(const U4& v, float mu) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(w[i]) - mu, hi = bf16_hi(w[i]) - mu;
    p[i] = lo * lo + hi * hi;
  }
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// fp64 sums (of the elements, then of the squared deviations from m) for
// rows whose fp32 sums leave the safe range. The words pass through an empty
// asm so their unpacking is not shared with (and hoisted above this branch
// for) the normalisation.
__device__ __forceinline__ double sum_u4_f64(const U4& v, double s) {
  uint32_t d[4] = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (double)bf16_lo(d[i]) + (double)bf16_hi(d[i]);
  return s;
}
__device__ __forceinline__ double sqdev_u4_f64(const U4& v, double m, double ss) {
  uint32_t d[4] = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = (double)bf16_lo(d[i]) - m, b = (double)bf16_hi(d[i]) - m;
    ss = __builtin_fma(a, a, ss);
    ss = __builtin_fma(b, b, ss);
  }
  return ss;
}

// y and the modulation for eight elements (pairs stay packed as BF16). The
// affine step and the modulation are compile-time choices; a missing half of
// either comes in as its identity (gamma 1, beta 0, m 1, shift 0), which
// changes nothing but the sign of a zero, and no code depends on that. m is
// the packed bf16(fl32(1 + scale)), formed once per workgroup.
template <bool kAffine, bool kMod>
__device__ __forceinline__ U4 layernorm_u4(const U4& v, float mu, float r, const U4& g,
                                           const U4& b, const U4& m, const U4& sh) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, bw[4] = {b.x, b.y, b.z, b.w};
  const uint32_t mw[4] = {m.x, m.y, m.z, m.w}, hw[4] = {sh.x, sh.y, sh.z, sh.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = (bf16_lo(d[i]) - mu) * r;
    float hi = (bf16_hi(d[i]) - mu) * r;
    if constexpr (kAffine) {
      lo = lo * bf16_lo(gw[i]) + bf16_lo(bw[i]);
      hi = hi * bf16_hi(gw[i]) + bf16_hi(bw[i]);
    }
    uint32_t y = pack_bf16x2(lo, hi);
    if constexpr (kMod) {
      y = pack_bf16x2(bf16_lo(y) * bf16_lo(mw[i]), bf16_hi(y) * bf16_hi(mw[i]));
      y = pack_bf16x2(bf16_lo(y) + bf16_lo(hw[i]), bf16_hi(y) + bf16_hi(hw[i]));
    }
    o[i] = y;
  }
  return U4{o[0], o[1], o[2], o[3]};
}

// packed bf16(fl32(1 + scale)) of a vector of scale pairs
__device__ __forceinline__ U4 one_plus_bf16(const U4& c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(1.0f + bf16_lo(w[i]), 1.0f + bf16_hi(w[i]));
  return U4{o[0], o[1], o[2], o[3]};
}

constexpr int kLnRowsPerBlock = 8;   // rows (waves) sharing the staged vectors

// 16-byte vector idx of an optional [cols] BF16 vector, or its identity value.
__device__ __forceinline__ U4 opt_vec(const U4* p, int idx, uint32_t identity) {
  return p ? p[idx] : U4{identity, identity, identity, identity};
}

// ---------------------------------------------------------------------------
// Rows of up to 640 vectors (K <= 5120): the row is held as fp32 deviations
// x - mu, formed once for the variance and reused by the normalisation, and
// every BF16 rounding of the chain is one v_cvt_pk_bf16_f32 whose result is
// already the rounded fp32 value (round_bf16), so no value is unpacked twice.
// The per-channel vectors are staged in LDS as fp32 (m = bf16(1 + scale)
// formed there), split into two 16-byte halves per 8-channel vector so each
// ds_read_b128 of a wave reads 1 KiB of consecutive LDS.
// ---------------------------------------------------------------------------
constexpr int kLnF32MaxVpl = 10;
// Rows per workgroup: 8 (two waves per SIMD), 4 for rows of 10 vectors per
// lane, whose registers leave room for three waves per SIMD.
template <int kVpl>
constexpr int ln_rows_per_block() { return kVpl > 8 ? 4 : 8; }

// 1 / sqrt(a) in fp64: v_rsq_f64, then two Newton steps y (3 - a y^2) / 2,
// each of which squares the relative error, for a positive finite a (zero
// and infinity keep the first estimate, inf and 0). The result is within a
// few fp64 ulps of the exact value, so its fp32 rounding is the correctly
// rounded one unless the exact value lies within about 2^-50 (relative) of a
// rounding boundary, and then it is the other neighbour.
__device__ __forceinline__ double rsqrt_f64(double a) {
  double y = __builtin_amdgcn_rsq(a);
  const double h = 0.5 * a;
#pragma unroll
  for (int it = 0; it < 2; ++it) y = y * __builtin_fma(-h * y, y, 1.5);
  return (a > 0.0 && a < __builtin_inf()) ? y : __builtin_amdgcn_rsq(a);
}
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const U4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// Sum of the eight squares, two fma chains of four then one add (depth 5
// counting the first product's rounding).
__device__ __forceinline__ float sumsq8_dev(const float (&d)[8]) {
  float a = d[0] * d[0], b = d[4] * d[4];
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    a = __builtin_fmaf(d[e], d[e], a);
    b = __builtin_fmaf(d[e + 4], d[e + 4], b);
  }
  return a + b;
}

// Eight fp32 values (each exactly a BF16 value) -> eight INT8 codes.
template <bool kFast>
__device__ __forceinline__ uint2 quant_f8(const float (&z)[8], const QuantParams& p) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = quant_quotient<kFast>(z[e], p);
  return make_uint2(code_bytes4<kFast>(t[0], t[1], t[2], t[3]),
                    code_bytes4<kFast>(t[4], t[5], t[6], t[7]));
}

template <int kVpl, bool kFull, bool kAffine, bool kMod, int kRows>
__global__ __launch_bounds__(kRows * kWave)
void layernorm_quant_f32_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                const uint16_t* __restrict__ beta,
                                const uint16_t* __restrict__ mod_scale,
                                const uint16_t* __restrict__ mod_shift, float eps, int64_t rows,
                                int64_t cols, double inv_cols, int64_t ldx,
                                int8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale,
                                float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  static_assert(kVpl <= kLnF32MaxVpl, "fp32-resident rows hold at most 10 vectors per lane");
  constexpr int kStaged = (kAffine ? 2 : 0) + (kMod ? 2 : 0);
  constexpr int kSlots = kVpl * kWave;
  // [staged vector][half][slot]: channels 8 slot + 4 half + 0..3
  __shared__ v4f staged[kStaged > 0 ? kStaged : 1][2][kSlots];
  const int lane = threadIdx.x & (kWave - 1);
  const int nvec = (int)(cols >> 3);
  // Persistent: wave w of workgroup b takes rows b * kRows + w + k * (kRows * grid).
  const int64_t stride = (int64_t)gridDim.x * kRows;
  int64_t row = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if constexpr (kStaged > 0) {
    const U4* gr = reinterpret_cast<const U4*>(gamma);
    const U4* br = reinterpret_cast<const U4*>(beta);
    const U4* cr = reinterpret_cast<const U4*>(mod_scale);
    const U4* hr = reinterpret_cast<const U4*>(mod_shift);
    const auto put = [&](int t, int i, const float (&f)[8]) {
      staged[t][0][i] = v4f{f[0], f[1], f[2], f[3]};
      staged[t][1][i] = v4f{f[4], f[5], f[6], f[7]};
    };
    for (int i = threadIdx.x; i < kSlots; i += kRows * kWave) {
      const int idx = i < nvec ? i : nvec - 1;
      float f[8];
      int t = 0;
      if constexpr (kAffine) {
        unpack8(opt_vec(gr, idx, kBf16OnePair), f);
        put(t++, i, f);
        unpack8(opt_vec(br, idx, 0u), f);
        put(t++, i, f);
      }
      if constexpr (kMod) {
        unpack8(opt_vec(cr, idx, 0u), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = round_bf16(1.0f + f[e]);
        put(t++, i, f);
        unpack8(opt_vec(hr, idx, 0u), f);
        put(t++, i, f);
      }
    }
    __syncthreads();
  }
  for (; row < rows; row += stride) {
    U4 v[kVpl];
    load_row<kVpl, kFull>(v, reinterpret_cast<const U4*>(x + row * ldx), lane, nvec);
    // Mean from pairwise fp32 sums (depth 3 per vector, then the vectors and
    // the wave), then the deviations d = fl32(x - mu), whose squares give the
    // variance; padding vectors are left out of it. Each sum is within about
    // (log2(cols) + 7) * 2^-24 of the exact one, relative to the sum of |x|
    // and to the sum of squares respectively. A row whose fp32 sum overflows
    // takes its mean from an fp64 sum; one whose sum of squares overflows or
    // falls below 2^-80 (squares in the subnormal range) sums the squares of
    // the same deviations in fp64. Both choices are uniform over the wave and
    // leave d where it is.
    float part[kVpl];
#pragma unroll
    for (int j = 0; j < kVpl; ++j) part[j] = sum8_f32(v[j]);
    const float s1 = wave_sum_f32(tree_sum<0, kVpl>(part));
    float mu;
    if (__builtin_isfinite(s1)) {
      mu = (float)((double)s1 * inv_cols);
    } else {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < kVpl; ++j) s = sum_u4_f64(v[j], s);   // padding vectors are zero
      mu = (float)(wave_sum_f64(s) * inv_cols);
    }
    float d[kVpl][8];
#pragma unroll
    for (int j = 0; j < kVpl; ++j) {
      unpack8(v[j], d[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) d[j][e] -= mu;
      part[j] = has_vec<kVpl, kFull>(lane, j, nvec) ? sumsq8_dev(d[j]) : 0.0f;
    }
    const float s2 = wave_sum_f32(tree_sum<0, kVpl>(part));
    double var;
    if (s2 >= 0x1p-80f && s2 <= 0x1p126f) {
      var = (double)s2 * inv_cols;
    } else {
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < kVpl; ++j)
        if (has_vec<kVpl, kFull>(lane, j, nvec))
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)d[j][e], (double)d[j][e], ss);
      var = wave_sum_f64(ss) * inv_cols;
    }
    const float r = (float)rsqrt_f64(var + (double)eps);
    // normalise, affine step, modulation; the row's absmax
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) {
      const int i = lane + j * kWave;
      float st[kStaged > 0 ? kStaged : 1][8];
#pragma unroll
      for (int t = 0; t < kStaged; ++t) {
        const v4f a = staged[t][0][i], b = staged[t][1][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st[t][e] = a[e];
          st[t][e + 4] = b[e];
        }
      }
      const bool in = has_vec<kVpl, kFull>(lane, j, nvec);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float u = d[j][e] * r;
        if constexpr (kAffine) {
          u = u * st[0][e];
          u = u + st[1][e];
        }
        float y = round_bf16(u);
        if constexpr (kMod) {
          y = round_bf16(y * st[kAffine ? 2 : 0][e]);
          y = round_bf16(y + st[kAffine ? 3 : 1][e]);
        }
        d[j][e] = in ? y : 0.0f;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(d[j][e]));
      }
      // keep the staged-vector reads to one vector ahead: the scheduler would
      // otherwise hoist them all and hold them with the whole row
      __builtin_amdgcn_sched_barrier(0);
    }
    // |y| as bits orders like the values (non-negative floats)
    const QuantParams p = quant_params(__uint_as_float(wave_max_u32(__float_as_uint(amax))));
    uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
    if (p.fast) {
#pragma unroll
      for (int j = 0; j < kVpl; ++j)
        if (has_vec<kVpl, kFull>(lane, j, nvec)) qr[lane + j * kWave] = quant_f8<true>(d[j], p);
    } else {
#pragma unroll
      for (int j = 0; j < kVpl; ++j)
        if (has_vec<kVpl, kFull>(lane, j, nvec)) qr[lane + j * kWave] = quant_f8<false>(d[j], p);
    }
    if (lane == 0) {
      scale[row] = p.s;
      if (mean_out) mean_out[row] = mu;
      if (rstd_out) rstd_out[row] = r;
    }
  }
}

// Workgroups of a persistent kernel resident at once on one CU (from its
// registers and LDS), queried once per kernel. Host threads may race to fill
// the cache with the same value; it is an atomic so that this is well defined.
template <typename Kernel>
static unsigned resident_per_cu(Kernel kernel, int block, std::atomic<int>& cache) {
  int n = cache.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) !=
            hipSuccess ||
        n < 1) {
      (void)hipGetLastError();   // the query's failure is not the launch's
      n = 1;
    }
    cache.store(n, std::memory_order_relaxed);
  }
  return (unsigned)n;
}

// Longer rows (K up to 8192): the row stays packed as BF16 between the steps.
template <int kVpl, bool kFull, bool kAffine, bool kMod>
__global__ __launch_bounds__(kLnRowsPerBlock * kWave)
void layernorm_quant_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                            const uint16_t* __restrict__ beta,
                            const uint16_t* __restrict__ mod_scale,
                            const uint16_t* __restrict__ mod_shift, float eps, int64_t rows,
                            int64_t cols, int64_t ldx, int8_t* __restrict__ q, int64_t ldq,
                            float* __restrict__ scale, float* __restrict__ mean_out,
                            float* __restrict__ rstd_out) {
  // The per-channel vectors of the affine step and the modulation, staged
  // once per workgroup in LDS (with m = bf16(1 + scale) formed here), so each
  // row reads them from LDS instead of L2.
  constexpr int kStaged = (kAffine ? 2 : 0) + (kMod ? 2 : 0);
  __shared__ __attribute__((aligned(16))) U4 staged[kStaged > 0 ? kStaged : 1][kVpl * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
  const int nvec = (int)(cols >> 3);
  U4 v[kVpl];
  if (row < rows)   // the row's loads go out first; the whole workgroup stages below
    load_row<kVpl, kFull>(v, reinterpret_cast<const U4*>(x + row * ldx), lane, nvec);
  if constexpr (kStaged > 0) {
    const U4* gr = reinterpret_cast<const U4*>(gamma);
    const U4* br = reinterpret_cast<const U4*>(beta);
    const U4* cr = reinterpret_cast<const U4*>(mod_scale);
    const U4* hr = reinterpret_cast<const U4*>(mod_shift);
    for (int i = threadIdx.x; i < kVpl * kWave; i += kLnRowsPerBlock * kWave) {
      const int idx = i < nvec ? i : nvec - 1;
      int t = 0;
      if constexpr (kAffine) {
        staged[t++][i] = opt_vec(gr, idx, kBf16OnePair);
        staged[t++][i] = opt_vec(br, idx, 0u);
      }
      if constexpr (kMod) {
        staged[t++][i] = one_plus_bf16(opt_vec(cr, idx, 0u));
        staged[t++][i] = opt_vec(hr, idx, 0u);
      }
    }
    __syncthreads();
  }
  if (row >= rows) return;
  // Statistics: the mean from pairwise fp32 sums of the elements, then the
  // sum of squared deviations about that fp32 mean (padding vectors left
  // out). Each is within about (log2(cols) + 6) * 2^-24 of the exact value,
  // relative to the sum of |x| and to the sum of squares respectively.
  float part[kVpl];
#pragma unroll
  for (int j = 0; j < kVpl; ++j) part[j] = sum8_f32(v[j]);
  const float s1 = wave_sum_f32(tree_sum<0, kVpl>(part));
  float mu = (float)((double)s1 / (double)cols);
#pragma unroll
  for (int j = 0; j < kVpl; ++j)
    part[j] = has_vec<kVpl, kFull>(lane, j, nvec) ? sqdev8_f32(v[j], mu) : 0.0f;
  const float s2 = wave_sum_f32(tree_sum<0, kVpl>(part));
  double var;
  if (__builtin_isfinite(s1) && s2 >= 0x1p-80f && s2 <= 0x1p100f) {
    var = (double)s2 / (double)cols;
  } else {
    double s = 0.0, ss = 0.0;
#pragma unroll
    for (int j = 0; j < kVpl; ++j) s = sum_u4_f64(v[j], s);   // padding vectors are zero
    const double m64 = wave_sum_f64(s) / (double)cols;
#pragma unroll
    for (int j = 0; j < kVpl; ++j)
      if (has_vec<kVpl, kFull>(lane, j, nvec)) ss = sqdev_u4_f64(v[j], m64, ss);
    var = wave_sum_f64(ss) / (double)cols;
    mu = (float)m64;
  }
  const float r = (float)(1.0 / __builtin_sqrt(var + (double)eps));
  // The row passes through an empty asm: otherwise the compiler keeps the
  // variance pass's x - mu values for the normalisation, all of the row's
  // differences live at once instead of its packed words.
#pragma unroll
  for (int j = 0; j < kVpl; ++j)
    asm volatile("" : "+v"(v[j].x), "+v"(v[j].y), "+v"(v[j].z), "+v"(v[j].w));
  // normalise, modulate
  uint32_t m2 = 0;
#pragma unroll
  for (int j = 0; j < kVpl; ++j) {
    const int i = lane + j * kWave;
    const U4 zero{0u, 0u, 0u, 0u};
    const U4 gv = kAffine ? staged[0][i] : zero;
    const U4 bv = kAffine ? staged[1][i] : zero;
    const U4 mv = kMod ? staged[kAffine ? 2 : 0][i] : zero;
    const U4 hv = kMod ? staged[kAffine ? 3 : 1][i] : zero;
    const U4 z = layernorm_u4<kAffine, kMod>(v[j], mu, r, gv, bv, mv, hv);
    v[j] = has_vec<kVpl, kFull>(lane, j, nvec) ? z : zero;
    m2 = absmax2_u4(v[j], m2);
    // keep the staged-vector reads to four vectors ahead: the scheduler would
    // otherwise hoist them all and hold them with the whole row
    if constexpr (kVpl >= 8)
      if (j % 4 == 3) __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t m = wave_max_u32(fold_absmax(m2));
  const QuantParams p = quant_params(bf16_bits_to_float(m));
  uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
  if (p.fast) store_row_codes<kVpl, kFull, true>(v, qr, lane, nvec, p);
  else store_row_codes<kVpl, kFull, false>(v, qr, lane, nvec, p);
  if (lane == 0) {
    scale[row] = p.s;
    if (mean_out) mean_out[row] = mu;
    if (rstd_out) rstd_out[row] = r;
  }
}

template <int kVpl, bool kFull, bool kAffine, bool kMod>
static void launch_layernorm_variant(dim3 grid, dim3 block, hipStream_t st, const uint16_t* x,
                                     const uint16_t* gamma, const uint16_t* beta,
                                     const uint16_t* mod_scale, const uint16_t* mod_shift,
                                     float eps, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                                     int64_t ldq, float* scale, float* mean, float* rstd) {
  if constexpr (kVpl <= kLnF32MaxVpl) {
    // persistent: as many workgroups as are resident at once (from the
    // variant's registers and LDS), each wave looping over its rows
    constexpr int kRows = ln_rows_per_block<kVpl>();
    static std::atomic<int> per_cu{0};
    const unsigned resident =
        resident_per_cu(layernorm_quant_f32_kernel<kVpl, kFull, kAffine, kMod, kRows>,
                        kRows * kWave, per_cu) *
        (unsigned)device_cu_count();
    const unsigned need = (unsigned)((rows + kRows - 1) / kRows);
    hipLaunchKernelGGL((layernorm_quant_f32_kernel<kVpl, kFull, kAffine, kMod, kRows>),
                       dim3(need < resident ? need : resident), dim3(kRows * kWave), 0, st, x,
                       gamma, beta, mod_scale, mod_shift, eps, rows, cols, 1.0 / (double)cols,
                       ldx, q, ldq, scale, mean, rstd);
  }
  else
    hipLaunchKernelGGL((layernorm_quant_kernel<kVpl, kFull, kAffine, kMod>), grid, block, 0, st, x,
                       gamma, beta, mod_scale, mod_shift, eps, rows, cols, ldx, q, ldq, scale,
                       mean, rstd);
}

template <int kVpl, bool kFull>
static hipError_t launch_layernorm(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                                   const uint16_t* mod_scale, const uint16_t* mod_shift,
                                   float eps, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                                   int64_t ldq, float* scale, float* mean, float* rstd,
                                   hipStream_t st) {
  const dim3 grid((unsigned)((rows + kLnRowsPerBlock - 1) / kLnRowsPerBlock));
  const dim3 block(kLnRowsPerBlock * kWave);
  const bool affine = gamma || beta, mod = mod_scale || mod_shift;
#define W8A8_LN_LAUNCH(A, M)                                                                  \
  launch_layernorm_variant<kVpl, kFull, A, M>(grid, block, st, x, gamma, beta, mod_scale,    \
                                              mod_shift, eps, rows, cols, ldx, q, ldq, scale, \
                                              mean, rstd)
  if (affine && mod) W8A8_LN_LAUNCH(true, true);
  else if (affine) W8A8_LN_LAUNCH(true, false);
  else if (mod) W8A8_LN_LAUNCH(false, true);
  else W8A8_LN_LAUNCH(false, false);
#undef W8A8_LN_LAUNCH
  return hipGetLastError();
}

template <int kVpl, bool kFull>
static hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t rows,
                                 int64_t cols, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                 float* inv_rms, hipStream_t st) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((rmsnorm_quant_kernel<kVpl, kFull>), grid, dim3(kRowsPerBlock * kWave), 0, st,
                     x, gamma, eps, rows, cols, ldx, q, ldq, scale, inv_rms);
  return hipGetLastError();
}

template <int kVpl, bool kG128, bool kFull>
static hipError_t launch_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int8_t* q,
                              int64_t ldq, float* scale, hipStream_t st) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((quant_rows_kernel<kVpl, kG128, kFull>), grid, dim3(kRowsPerBlock * kWave), 0,
                     st, x, rows, cols, ldx, q, ldq, scale);
  return hipGetLastError();
}

// Register-resident variants: vectors per lane. A row of nvec vectors takes
// the smallest variant that holds it, the exact ("full", unpredicated) one
// when nvec is a multiple of 64 in this list: K = 4096, 5120, 6144, 8192,
// 13824 and 16384 all are.
static int pick_vpl(int64_t nvec) {
  static const int kChoices[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 14, 16, 20, 24, 27, 28, 32};
  for (int c : kChoices)
    if (nvec <= (int64_t)c * kWave) return c;
  return 0;
}

// The few-rows kernel: up to kSplitRowsMax rows (fewer than 4 waves per SIMD
// with one wave per row). Per-token rows take it from 1024 vectors (8192
// columns) on, where one wave's chain over the row is long; below that it
// gains nothing (graph-replayed on MI355X: 1000 x 5120 in 3.5 us either way,
// 256 x 13824 in 5.1 us one wave per row against 3.2 us, 1000 x 8192 5.6
// against 4.6 us). (1, 128) groups need no barrier and take it from 128
// vectors on (1000 x 5120: 4.5 against 3.6 us). Its shape: the fewest waves
// per row (2 to 16) whose vectors-per-lane count, 4 down to 1, covers the row
// exactly (10 waves of 1 vector took 6.4 us at 1000 x 5120, 5 waves of 2
// about the single-wave time), else 8 waves with the predicated variant.
constexpr int64_t kSplitRowsMax = 2048;
struct SplitShape {
  int waves, vpl;
  bool full;
};
static SplitShape pick_split(int64_t nvec, bool g128) {
  if (nvec < (g128 ? 2 : 16) * kWave || nvec > (int64_t)kMaxSplitWaves * 4 * kWave)
    return {0, 0, false};
  for (int v = 4; v >= 1; --v)
    for (int wv = 2; wv <= kMaxSplitWaves; ++wv)
      if ((int64_t)wv * v * kWave == nvec) return {wv, v, true};
  const int64_t per = 8 * kWave;
  const int v = (int)((nvec + per - 1) / per);
  return v <= 4 ? SplitShape{8, v, false} : SplitShape{0, 0, false};
}

#define W8A8_VPL_CASE(V, CALL) \
  case V: return full ? CALL(V, true) : CALL(V, false);
#define W8A8_VPL_SWITCH(VPL, CALL)                                                   \
  switch (VPL) {                                                                     \
    W8A8_VPL_CASE(1, CALL) W8A8_VPL_CASE(2, CALL) W8A8_VPL_CASE(3, CALL)             \
    W8A8_VPL_CASE(4, CALL) W8A8_VPL_CASE(5, CALL) W8A8_VPL_CASE(6, CALL)             \
    W8A8_VPL_CASE(8, CALL) W8A8_VPL_CASE(10, CALL) W8A8_VPL_CASE(12, CALL)           \
    W8A8_VPL_CASE(14, CALL) W8A8_VPL_CASE(16, CALL) W8A8_VPL_CASE(20, CALL)          \
    W8A8_VPL_CASE(24, CALL) W8A8_VPL_CASE(27, CALL) W8A8_VPL_CASE(28, CALL)          \
    W8A8_VPL_CASE(32, CALL)                                                          \
    default: break;                                                                  \
  }

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             int64_t group_rows, int64_t group_cols, int8_t* q, int64_t ldq,
                             float* scale, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (group_rows == 128) {
    const dim3 grid((unsigned)(cols >> 7), (unsigned)((rows + 127) / 128));
    hipLaunchKernelGGL(quant_block128_kernel, grid, dim3(256), 0, st, x, rows, cols, ldx, q, ldq,
                       scale);
    return hipGetLastError();
  }
  // (1, 128) on a 128-wide matrix is the same as one group per row
  const bool g128 = group_cols == 128 && cols != 128;
  if (rows <= kSplitRowsMax) {
    const SplitShape sp = pick_split(cols >> 3, g128);
    if (sp.waves > 0) {
#define W8A8_SPLIT(V, G, F)                                                                  \
  hipLaunchKernelGGL((quant_rows_split_kernel<V, G, F>), dim3((unsigned)rows),               \
                     dim3(sp.waves * kWave), 0, st, x, cols, ldx, q, ldq, scale);             \
  return hipGetLastError();
#define W8A8_SPLIT_F(V, G) \
  if (sp.full) { W8A8_SPLIT(V, G, true) } else { W8A8_SPLIT(V, G, false) }
#define W8A8_SPLIT_G(V) \
  if (g128) { W8A8_SPLIT_F(V, true) } else { W8A8_SPLIT_F(V, false) }
      switch (sp.vpl) {
        case 1: { W8A8_SPLIT_G(1) }
        case 2: { W8A8_SPLIT_G(2) }
        case 3: { W8A8_SPLIT_G(3) }
        case 4: { W8A8_SPLIT_G(4) }
        default: break;
      }
#undef W8A8_SPLIT_G
#undef W8A8_SPLIT_F
#undef W8A8_SPLIT
    }
  }
  const int vpl = pick_vpl(cols >> 3);
  const bool full = vpl > 0 && (cols >> 3) == (int64_t)vpl * kWave;
  if (!g128) {
#define W8A8_CALL_ROW(V, F) launch_rows<V, false, F>(x, rows, cols, ldx, q, ldq, scale, st)
    W8A8_VPL_SWITCH(vpl, W8A8_CALL_ROW)
#undef W8A8_CALL_ROW
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    hipLaunchKernelGGL((quant_rows_long_kernel<false>), grid, dim3(kRowsPerBlock * kWave), 0, st,
                       x, rows, cols, ldx, q, ldq, scale);
    return hipGetLastError();
  }
#define W8A8_CALL_G128(V, F) launch_rows<V, true, F>(x, rows, cols, ldx, q, ldq, scale, st)
  W8A8_VPL_SWITCH(vpl, W8A8_CALL_G128)
#undef W8A8_CALL_G128
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((quant_rows_long_kernel<true>), grid, dim3(kRowsPerBlock * kWave), 0, st, x,
                     rows, cols, ldx, q, ldq, scale);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t rows,
                                int64_t cols, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                float* inv_rms, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int vpl = pick_vpl(cols >> 3);
  const bool full = vpl > 0 && (cols >> 3) == (int64_t)vpl * kWave;
#define W8A8_CALL_RMS(V, F) \
  launch_rmsnorm<V, F>(x, gamma, eps, rows, cols, ldx, q, ldq, scale, inv_rms, st)
  W8A8_VPL_SWITCH(vpl, W8A8_CALL_RMS)
#undef W8A8_CALL_RMS
  return hipErrorInvalidValue;   // host validation rejects longer rows first
}

hipError_t launch_layernorm_quant(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                                  const uint16_t* mod_scale, const uint16_t* mod_shift, float eps,
                                  int64_t rows, int64_t cols, int64_t ldx, int8_t* q, int64_t ldq,
                                  float* scale, float* mean, float* rstd, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  // vectors per lane: the smallest of 1, 2, 3, 4, 5, 6, 8, 10, 12, 16 that
  // holds the row (the common widths 1536, 2560, 3072, 4096, 5120 and 8192
  // are exact, unpredicated rows; others run masked)
  const int64_t nvec = cols >> 3;
  static const int kLnChoices[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
  int vpl = 0;
  for (int c : kLnChoices)
    if (vpl == 0 && nvec <= (int64_t)c * kWave) vpl = c;
  const bool full = nvec == (int64_t)vpl * kWave;
#define W8A8_CALL_LN(V, F)                                                                  \
  launch_layernorm<V, F>(x, gamma, beta, mod_scale, mod_shift, eps, rows, cols, ldx, q, ldq, \
                         scale, mean, rstd, st)
  switch (vpl) {
    W8A8_VPL_CASE(1, W8A8_CALL_LN) W8A8_VPL_CASE(2, W8A8_CALL_LN)
    W8A8_VPL_CASE(3, W8A8_CALL_LN) W8A8_VPL_CASE(4, W8A8_CALL_LN)
    W8A8_VPL_CASE(5, W8A8_CALL_LN) W8A8_VPL_CASE(6, W8A8_CALL_LN)
    W8A8_VPL_CASE(8, W8A8_CALL_LN) W8A8_VPL_CASE(10, W8A8_CALL_LN)
    W8A8_VPL_CASE(12, W8A8_CALL_LN) W8A8_VPL_CASE(16, W8A8_CALL_LN)
    default: break;
  }
#undef W8A8_CALL_LN
  return hipErrorInvalidValue;   // host validation rejects longer rows first
}

}  // namespace w8a8
