// Dispatch of the INT8 x INT8 GEMM epilogues to their kernels.
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", W8A8-kernel row and the paragraph under the table: the
// post-scale kernel keeps one INT32 accumulation over all of K and applies the
// activation and weight scales only in the epilogue (gemm_pipelined.hip; the
// INT32 export shares its main loop; split-K for small grids in splitk.hip);
// the original TurboDiffusion kernel rescales per K block (gemm_blockwise.hip).
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
      return launch_gemm_pipelined(epi, a, lda, w, ldw, a_scale, w_scale, bias, out, ldo, M, N, K,
                                   st);
    }
    case Epilogue::kInt32:
      return launch_gemm_pipelined(epi, a, lda, w, ldw, a_scale, w_scale, bias, out, ldo, M, N, K,
                                   st);
    case Epilogue::kBlockwiseBf16:
      return launch_gemm_blockwise(a, lda, w, ldw, a_scale, w_scale,
                                   reinterpret_cast<uint16_t*>(out), ldo, M, N, K, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace w8a8
