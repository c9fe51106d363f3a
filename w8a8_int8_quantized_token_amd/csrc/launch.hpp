// Internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Longest row the register-resident RMSNorm kernel holds (32 vectors of
// eight BF16 per lane, 64 lanes).
constexpr int64_t kRmsnormMaxCols = 32 * 64 * 8;
// ... and the LayerNorm kernel (16 vectors per lane; DiT hidden sizes are
// 4096 and 5120).
constexpr int kLayernormMaxVpl = 16;
constexpr int64_t kLayernormMaxCols = kLayernormMaxVpl * 64 * 8;

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                             int64_t group_rows, int64_t group_cols, int8_t* q, int64_t ldq,
                             float* scale, hipStream_t st);

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t rows,
                                int64_t cols, int64_t ldx, int8_t* q, int64_t ldq, float* scale,
                                float* inv_rms, hipStream_t st);

hipError_t launch_layernorm_quant(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta,
                                  const uint16_t* mod_scale, const uint16_t* mod_shift, float eps,
                                  int64_t rows, int64_t cols, int64_t ldx, int8_t* q, int64_t ldq,
                                  float* scale, float* mean, float* rstd, hipStream_t st);

enum class Epilogue {
  kPostscaleBf16,
  kInt32,
  kBlockwiseBf16,
  kPostscaleBiasBf16,
  kPostscaleGeluBf16,       // GELU of the BF16 post-scale output
  kPostscaleBiasGeluBf16,   // GELU of the BF16 post-scale-plus-bias output
};
constexpr bool epilogue_has_bias(Epilogue e) {
  return e == Epilogue::kPostscaleBiasBf16 || e == Epilogue::kPostscaleBiasGeluBf16;
}
constexpr bool epilogue_has_gelu(Epilogue e) {
  return e == Epilogue::kPostscaleGeluBf16 || e == Epilogue::kPostscaleBiasGeluBf16;
}

// Compute units of the current device (cached per device); persistent grids
// launch at most one workgroup per CU.
int device_cu_count();

// Persistent pipelined kernel (post-scale and INT32 epilogues). With
// splits > 1 (INT32 only, splits <= K / 128) K is cut into `splits` parts of
// whole 128-byte stages and part p's sums go to out + p * M * ldo.
hipError_t launch_gemm_pipelined(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w,
                                 int64_t ldw, const float* a_scale, const float* w_scale,
                                 const uint16_t* bias, void* out, int64_t ldo, int64_t M,
                                 int64_t N, int64_t K, hipStream_t st, int splits = 1);

// out[m, n] = bf16(fl32(fl32(fl32(sum_p part_p[m, n]) * a_scale[m]) * w_scale[n])
// (+ bias[n])), then with gelu its GELU rounded to BF16: the post-scale
// epilogue over INT32 partial sums part_p = ws + p * M * N (each [M, N], row
// stride N).
hipError_t launch_splitk_postscale(const int32_t* ws, int splits, int64_t M, int64_t N,
                                   const float* a_scale, const float* w_scale,
                                   const uint16_t* bias, bool gelu, uint16_t* out, int64_t ldo,
                                   hipStream_t st);

// Split-K limits: at most this many K parts, and the library's own choice
// never asks for a larger workspace than this (bytes).
constexpr int kMaxSplitParts = 64;
constexpr int64_t kMaxSplitWorkspace = (int64_t)1 << 30;

// K parts for a post-scale GEMM of this shape on `cus` compute units, from a
// cost model of the split (fewer stages per work item against a per-item
// cost, the partial sums' traffic, a fixed cost and the host's floor); 1
// unless splitting saves 15% of the time. Only part counts whose partial sums
// fit max_ws bytes are considered. A pure function of its arguments.
int splitk_parts(int64_t M, int64_t N, int64_t K, int cus, int64_t max_ws = kMaxSplitWorkspace);

// 128-token x 160-channel tiles, one workgroup per tile (gemm_tile160.hip):
// the post-scale epilogues (bias, GELU) and the blockwise one. N % 128 == 0.
hipError_t launch_gemm_tile160(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w,
                               int64_t ldw, const float* a_scale, const float* w_scale,
                               const uint16_t* bias, uint16_t* out, int64_t ldo, int64_t M,
                               int64_t N, int64_t K, hipStream_t st);
int tile160_tiles(int64_t M, int64_t N);

// Estimated microseconds of one pass of the persistent kernels (256 x 256
// post-scale tiles, 256 x 128 blockwise tiles) and of the 128 x 160 kernel on
// `cus` compute units, and the choice between them: a single pass uses
// 128 x 160 tiles when that is estimated at least 10% faster (few tokens:
// the larger tiles leave compute units idle).
double single_pass_us_256(int64_t M, int64_t N, int64_t K, int cus, bool blockwise);
double single_pass_us_160(int64_t M, int64_t N, int64_t K, int cus, bool blockwise);
bool use_tile160(int64_t M, int64_t N, int64_t K, int cus, bool blockwise);

// Persistent pipelined kernel with per-K-block scales.
hipError_t launch_gemm_blockwise(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                 const float* a_scale, const float* w_scale, uint16_t* out,
                                 int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st);

// bias (BF16 [N]) is read by the bias epilogues only. A post-scale epilogue
// with parts > 1 runs split-K: the INT32 partial sums of the parts go to the
// caller's workspace ws (parts * M * N int32, 16-byte aligned), then one pass
// adds them and applies the epilogue; parts == 1 is the single pass.
hipError_t launch_gemm(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                       const float* a_scale, const float* w_scale, const uint16_t* bias,
                       void* out, int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st,
                       int parts = 1, void* ws = nullptr);

}  // namespace w8a8
