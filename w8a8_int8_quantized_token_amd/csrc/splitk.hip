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
// one 16-byte store. The partial sums are read once, with ordinary loads: the
// partial-sum pass has just written them and they are still in the caches
// (non-temporal loads took about 1 us longer at 256 x 5120 in 8 parts).
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
    v4i s0 = *reinterpret_cast<const v4i*>(src);
    v4i s1 = *reinterpret_cast<const v4i*>(src + 4);
    // unrolled so that several parts' loads are in flight at once: with few
    // outputs the grid is small and each part's loads would otherwise wait
    // out a full memory round trip
#pragma unroll 8
    for (int p = 1; p < splits; ++p) {
      s0 += *reinterpret_cast<const v4i*>(src + p * slice);
      s1 += *reinterpret_cast<const v4i*>(src + p * slice + 4);
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

int splitk_parts(int64_t M, int64_t N, int64_t K, int cus, int64_t max_ws) {
  const int64_t nk = K / 128;
  const int64_t bytes_per_part = M * N * 4;
  // Cost model in microseconds, fitted to timings of split and single passes
  // on MI355X (M from 64 to 2048, N from 1024 to 16384, K from 4096 to 13824,
  // 1 to 24 parts):
  //  * single pass: the better of the two tilings (gemm.hip);
  //  * split: per round of work items, 1.3 per stage plus 3 for the item's
  //    prologue and INT32 epilogue; 11 for the extra pass and the workspace;
  //    0.286 per MB of partial sums (written once, read once); and never
  //    below 25 (the fit's floor, measured when each split call also took
  //    and released its workspace on the stream).
  // Split only if that saves 15%, and then take the fewest parts within 5%
  // of the best (fewer partial bytes, same predicted time).
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const double stage_us = 1.3, item_us = 3.0, fixed_us = 11.0, us_per_byte = 0.286e-6,
               floor_us = 25.0;
  // the single pass on the better of its two tilings
  const double s256 = single_pass_us_256(M, N, K, cus, false);
  const double s160 = single_pass_us_160(M, N, K, cus, false);
  const double single = s160 < s256 ? s160 : s256;
  double est[kMaxSplitParts + 1] = {0};
  double best_us = 0.0;
  int64_t last = 1;
  for (int64_t parts = 2; parts <= nk && parts <= kMaxSplitParts; ++parts) {
    if (parts * bytes_per_part > max_ws) break;
    const double rounds = (double)((tiles * parts + cus - 1) / cus);
    double us = rounds * ((double)((nk + parts - 1) / parts) * stage_us + item_us) + fixed_us +
                us_per_byte * (double)(parts * bytes_per_part);
    us = us > floor_us ? us : floor_us;
    est[parts] = us;
    if (last == 1 || us < best_us) best_us = us;
    last = parts;
  }
  if (last == 1 || best_us >= 0.85 * single) return 1;
  int best = 1;
  for (int64_t parts = 2; parts <= last; ++parts)
    if (est[parts] <= 1.05 * best_us) {
      best = (int)parts;
      break;
    }
  return best;
}

}  // namespace w8a8
