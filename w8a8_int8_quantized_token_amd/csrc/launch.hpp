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

enum class Epilogue { kPostscaleBf16, kInt32, kBlockwiseBf16, kPostscaleBiasBf16 };

// Compute units of the current device (cached per device); persistent grids
// launch at most one workgroup per CU.
int device_cu_count();

// Persistent pipelined kernel (post-scale and INT32 epilogues).
hipError_t launch_gemm_pipelined(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w,
                                 int64_t ldw, const float* a_scale, const float* w_scale,
                                 const uint16_t* bias, void* out, int64_t ldo, int64_t M,
                                 int64_t N, int64_t K, hipStream_t st);

// Persistent pipelined kernel with per-K-block scales.
hipError_t launch_gemm_blockwise(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                 const float* a_scale, const float* w_scale, uint16_t* out,
                                 int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st);

// bias (BF16 [N]) is read by the kPostscaleBiasBf16 epilogue only.
hipError_t launch_gemm(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                       const float* a_scale, const float* w_scale, const uint16_t* bias,
                       void* out, int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st);

}  // namespace w8a8
