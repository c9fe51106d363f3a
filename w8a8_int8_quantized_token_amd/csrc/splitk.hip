// Split-K for post-scale GEMMs whose tiles do not fill the chip.
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", paragraph under the table: one INT32 accumulation over all
// of K, scales applied in the epilogue. Integer addition is exact and
// associative, so K may be cut into parts whose INT32 partial sums (from the
// pipelined kernel's INT32 epilogue) add up to exactly the full sum; this
// kernel adds them and applies the same fp32 epilogue (and GELU), in the same
// order, as the single-pass kernel, so the output is bit-identical to it.
//
// One thread per 8 consecutive outputs of a row: per part two 16-byte loads,
// one 16-byte store. The partial sums are read once (non-temporal).
#include <cstdlib>

#include "launch.hpp"
#include "pipeline.hpp"

namespace w8a8 {
namespace splitk {

constexpr int kThreads = 256;

template <bool kBias, bool kGelu>
__global__ __launch_bounds__(kThreads)
void postscale_kernel(const int32_t* __restrict__ ws, int splits, int M, int N,
                      const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t slice = (int64_t)M * N;
  const int n8 = N / 8;
  const int64_t units = (int64_t)M * n8;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kThreads) {
    const int m = (int)(u / n8);
    const int n = (int)(u - (int64_t)m * n8) * 8;
    const int32_t* src = ws + (int64_t)m * N + n;
    v4i s0 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
    v4i s1 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + 4));
    for (int p = 1; p < splits; ++p) {
      s0 += __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + p * slice));
      s1 += __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + p * slice + 4));
    }
    const float sa = a_scale[m];
    float v[8];   // the scales are only 4-byte aligned: scalar loads
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = ((float)s0[e] * sa) * w_scale[n + e];
      v[4 + e] = ((float)s1[e] * sa) * w_scale[n + 4 + e];
    }
    if constexpr (kBias) {
      const v4u b = *reinterpret_cast<const v4u*>(bias + n);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = v[2 * q] + bf16_lo(b[q]);
        v[2 * q + 1] = v[2 * q + 1] + bf16_hi(b[q]);
      }
    }
    if constexpr (kGelu) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = gelu_erf(round_bf16(v[e]));
    }
    __builtin_nontemporal_store(v4u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                reinterpret_cast<v4u*>(out + (int64_t)m * ldo + n));
  }
}

}  // namespace splitk

hipError_t launch_splitk_postscale(const int32_t* ws, int splits, int64_t M, int64_t N,
                                   const float* a_scale, const float* w_scale,
                                   const uint16_t* bias, bool gelu, uint16_t* out, int64_t ldo,
                                   hipStream_t st) {
  if (splits < 1 || N % 8 != 0) return hipErrorInvalidValue;
  const int64_t units = M * (N / 8);
  if (units == 0) return hipSuccess;
  const int64_t want = (units + splitk::kThreads - 1) / splitk::kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int grid = (int)(want < cap ? want : cap);
#define W8A8_SPLITK_LAUNCH(B, G)                                                           \
  hipLaunchKernelGGL((splitk::postscale_kernel<B, G>), dim3(grid), dim3(splitk::kThreads), 0, \
                     st, ws, splits, (int)M, (int)N, a_scale, w_scale, bias, out, ldo)
  if (bias && gelu) W8A8_SPLITK_LAUNCH(true, true);
  else if (bias) W8A8_SPLITK_LAUNCH(true, false);
  else if (gelu) W8A8_SPLITK_LAUNCH(false, true);
  else W8A8_SPLITK_LAUNCH(false, false);
#undef W8A8_SPLITK_LAUNCH
  return hipGetLastError();
}

int splitk_parts(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t nk = K / 128;
  static const int forced = [] {
    const char* e = std::getenv("W8A8_SPLIT_K");
    return e ? std::atoi(e) : 0;
  }();
  const int64_t bytes_per_part = M * N * 4;
  constexpr int64_t kMaxWorkspace = (int64_t)1 << 30;
  if (forced > 0) {
    int64_t parts = forced < nk ? forced : nk;
    while (parts > 1 && parts * bytes_per_part > kMaxWorkspace) --parts;
    return (int)parts;
  }
  // Cost model in microseconds, from measurements on MI355X: a 128-byte K
  // stage of a 256 x 256 tile takes about 1.3; the partial sums cost their
  // write and read at about 4 TB/s; the extra pass and the workspace cost
  // about 15 in all. Split only where it saves a quarter of the time.
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const double stage_us = 1.3, bytes_per_us = 4.0e6, fixed_us = 15.0;
  const double single = (double)((tiles + cus - 1) / cus) * nk * stage_us;
  int best = 1;
  double best_us = 0.75 * single;
  for (int64_t parts = 2; parts <= nk && parts <= 64; ++parts) {
    if (parts * bytes_per_part > kMaxWorkspace) break;
    const double rounds = (double)((tiles * parts + cus - 1) / cus);
    const double us = rounds * (double)((nk + parts - 1) / parts) * stage_us +
                      (2.0 * parts + 0.5) * (double)bytes_per_part / bytes_per_us + fixed_us;
    if (us < best_us) {
      best_us = us;
      best = (int)parts;
    }
  }
  return best;
}

}  // namespace w8a8
