// Dispatch of the INT8 x INT8 GEMM epilogues to their kernels.
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", W8A8-kernel row and the paragraph under the table: the
// post-scale kernel keeps one INT32 accumulation over all of K and applies the
// activation and weight scales only in the epilogue (gemm_pipelined.hip; the
// INT32 export shares its main loop; split-K for small grids in splitk.hip);
// the original TurboDiffusion kernel rescales per K block (gemm_blockwise.hip).
// With about a thousand tokens both run on 128 x 160 tiles instead
// (gemm_tile160.hip), when a cost model of the two tilings prefers them.
#include "launch.hpp"

namespace w8a8 {

hipError_t launch_gemm(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                       const float* a_scale, const float* w_scale, const uint16_t* bias,
                       void* out, int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st,
                       int parts, void* ws) {
  if (M == 0) return hipSuccess;
  switch (epi) {
    case Epilogue::kPostscaleBf16:
    case Epilogue::kPostscaleBiasBf16:
    case Epilogue::kPostscaleGeluBf16:
    case Epilogue::kPostscaleBiasGeluBf16: {
      // K in parts: exact INT32 partial sums in the caller's workspace, then
      // one pass that adds them and applies the epilogue (bit-identical to
      // the single pass).
      if (parts > 1) {
        if (!ws) return hipErrorInvalidValue;
        hipError_t e = launch_gemm_pipelined(Epilogue::kInt32, a, lda, w, ldw, nullptr, nullptr,
                                             nullptr, ws, N, M, N, K, st, parts);
        if (e != hipSuccess) return e;
        return launch_splitk_postscale(static_cast<const int32_t*>(ws), parts, M, N, a_scale,
                                       w_scale, epilogue_has_bias(epi) ? bias : nullptr,
                                       epilogue_has_gelu(epi), reinterpret_cast<uint16_t*>(out),
                                       ldo, st);
      }
      if (use_tile160(M, N, K, device_cu_count(), false))
        return launch_gemm_tile160(epi, a, lda, w, ldw, a_scale, w_scale, bias,
                                   reinterpret_cast<uint16_t*>(out), ldo, M, N, K, st);
      return launch_gemm_pipelined(epi, a, lda, w, ldw, a_scale, w_scale, bias, out, ldo, M, N, K,
                                   st);
    }
    case Epilogue::kInt32:
      return launch_gemm_pipelined(epi, a, lda, w, ldw, a_scale, w_scale, bias, out, ldo, M, N, K,
                                   st);
    case Epilogue::kBlockwiseBf16:
      if (use_tile160(M, N, K, device_cu_count(), true))
        return launch_gemm_tile160(epi, a, lda, w, ldw, a_scale, w_scale, nullptr,
                                   reinterpret_cast<uint16_t*>(out), ldo, M, N, K, st);
      return launch_gemm_blockwise(a, lda, w, ldw, a_scale, w_scale,
                                   reinterpret_cast<uint16_t*>(out), ldo, M, N, K, st);
  }
  return hipErrorInvalidValue;
}

// Estimated microseconds of one pass, fitted to graph-replayed timings on
// MI355X (M 512 - 4096, N 640 - 16384, K 128 - 13824):
//  * 256 x 256 post-scale tiles, persistent: 1.3 per 128-byte K stage per
//    round of tiles over the compute units, 3 once;
//  * 256 x 128 blockwise tiles, persistent: 1.0 per stage per round, 3 once;
//  * 128 x 160 tiles, one workgroup per tile: per round of tiles 5 (the
//    prologue's first loads and the epilogue) plus 0.55 per stage
//    (post-scale) or 0.8 (blockwise: the per-block rescale).
double single_pass_us_256(int64_t M, int64_t N, int64_t K, int cus, bool blockwise) {
  const int64_t bm = blockwise ? 128 : 256;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + 255) / 256);
  return (double)((tiles + cus - 1) / cus) * (double)(K / 128) * (blockwise ? 1.0 : 1.3) + 3.0;
}

double single_pass_us_160(int64_t M, int64_t N, int64_t K, int cus, bool blockwise) {
  const int64_t tiles = tile160_tiles(M, N);
  return (double)((tiles + cus - 1) / cus) * (5.0 + (double)(K / 128) * (blockwise ? 0.8 : 0.55));
}

bool use_tile160(int64_t M, int64_t N, int64_t K, int cus, bool blockwise) {
  return single_pass_us_160(M, N, K, cus, blockwise) <
         0.9 * single_pass_us_256(M, N, K, cus, blockwise);
}

}  // namespace w8a8
