// C ABI of the W8A8 library: host-side validation, then a launch on the
// caller's stream. See include/w8a8.h for the contract of each entry point.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.hpp"
#include "w8a8.h"

namespace {

thread_local std::string g_last_error;

w8a8_status_t fail(w8a8_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w8a8_status_t ok() {
  g_last_error.clear();
  return W8A8_OK;
}

w8a8_status_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(W8A8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p + n) and [q, q + m) overlap?
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

// Bytes spanned by a row-major [rows, cols] matrix with row stride ld.
size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)((rows - 1) * ld + cols) * elem;
}

constexpr int64_t kMaxRows = 0x7FFFFFFF;

w8a8_status_t check_quant_common(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                 const void* q, int64_t ldq, const void* scale) {
  if (rows < 0 || cols < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "negative size");
  if (rows > kMaxRows) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "rows > 2^31-1");
  if (cols == 0) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols must be positive");
  if (ldx < cols || ldq < cols) return fail(W8A8_ERR_INVALID_ARGUMENT, "leading dimension < cols");
  if (cols % 8) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols %% 8 != 0");
  if (ldx % 8 || ldq % 8)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "ldx %% 8 and ldq %% 8 must be 0");
  if (rows == 0) return W8A8_OK;          // nothing is read or written: pointers may be null
  if (!x || !q || !scale) return fail(W8A8_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(x, 16) || !aligned(q, 16))
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "x and q must be 16-byte aligned");
  if (!aligned(scale, 4)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "scale must be 4-byte aligned");
  return W8A8_OK;
}

w8a8_status_t check_gemm_common(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                const void* out, int64_t ldo, size_t out_elem, int64_t M,
                                int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "negative size");
  if (lda < K || ldw < K || ldo < N)
    return fail(W8A8_ERR_INVALID_ARGUMENT, "leading dimension smaller than the row");
  if (K < 128 || K % 128) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "K must be a positive multiple of 128");
  if (K > W8A8_MAX_K) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "K > %d overflows INT32", W8A8_MAX_K);
  if (N < 128 || N % 128) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "N must be a positive multiple of 128");
  if (M > kMaxRows || N > kMaxRows) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "M or N > 2^31-1");
  if (lda % 16 || ldw % 16) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "lda and ldw must be multiples of 16");
  if ((ldo * (int64_t)out_elem) % 16)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "output rows must start 16-byte aligned");
  if (M == 0) return W8A8_OK;             // nothing is read or written: pointers may be null
  if (!a || !w || !out) return fail(W8A8_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(out, 16))
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "a, w and out must be 16-byte aligned");
  // Per-tile offsets are 32-bit: 256 rows of either operand or of the
  // output must span less than 2^31 bytes.
  if ((int64_t)256 * (lda > ldw ? lda : ldw) > 0x7FFFFFFF ||
      (int64_t)256 * ldo * (int64_t)out_elem > 0x7FFFFFFF)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "leading dimension too large");
  const size_t out_bytes = span_bytes(M, N, ldo, out_elem);
  if (overlap(out, out_bytes, a, span_bytes(M, K, lda, 1)) ||
      overlap(out, out_bytes, w, span_bytes(N, K, ldw, 1)))
    return fail(W8A8_ERR_INVALID_ARGUMENT, "output overlaps an input");
  return W8A8_OK;
}

// Parts a post-scale call runs with: `parts` == 0 asks for the library's
// choice (the split-K cost model), else exactly `parts`. Returns -1 if
// `parts` is out of range for K.
int resolve_parts(int64_t M, int64_t N, int64_t K, int32_t parts) {
  if (parts < 0 || parts > w8a8::kMaxSplitParts || parts > K / 128) return -1;
  if (parts > 0) return parts;
  if (M <= 0) return 1;
  return w8a8::splitk_parts(M, N, K, w8a8::device_cu_count());
}

// The whole post-scale family: validation, then the single pass or split-K
// into the caller's workspace.
w8a8_status_t postscale_call(const char* name, const int8_t* a, int64_t lda, const int8_t* w,
                             int64_t ldw, const float* a_scale, const float* w_scale,
                             const uint16_t* bias, bool gelu, uint16_t* out, int64_t ldo,
                             int64_t M, int64_t N, int64_t K, int32_t parts, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  w8a8_status_t st = check_gemm_common(a, lda, w, ldw, out, ldo, 2, M, N, K);
  if (st != W8A8_OK) return st;
  const int resolved = resolve_parts(M, N, K, parts);
  if (resolved < 0)
    return fail(W8A8_ERR_INVALID_ARGUMENT, "parts must be 0 (library's choice) or 1..%d and at most K/128",
                w8a8::kMaxSplitParts);
  if (workspace_bytes < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "negative workspace_bytes");
  if (M == 0) return ok();
  if (!a_scale || !w_scale) return fail(W8A8_ERR_INVALID_ARGUMENT, "null scale pointer");
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "scales must be 4-byte aligned");
  if (bias && !aligned(bias, 16)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "bias must be 16-byte aligned");
  const size_t ob = span_bytes(M, N, ldo, 2);
  if (overlap(out, ob, a_scale, (size_t)M * 4) || overlap(out, ob, w_scale, (size_t)N * 4) ||
      (bias && overlap(out, ob, bias, (size_t)N * 2)))
    return fail(W8A8_ERR_INVALID_ARGUMENT, "output overlaps a scale or the bias");
  int run_parts = resolved;
  if (resolved > 1) {
    if (M * N > ((int64_t)1 << 50)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "M * N too large to split");
    const int64_t need = (int64_t)resolved * M * N * 4;
    if (!workspace) {
      // the library's own choice falls back to the single pass; parts the
      // caller asked for need the workspace
      if (parts > 1)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "%d parts need a workspace of %lld bytes",
                    resolved, (long long)need);
      run_parts = 1;
    } else {
      if (workspace_bytes < need)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "workspace of %lld bytes, %d parts need %lld",
                    (long long)workspace_bytes, resolved, (long long)need);
      if (!aligned(workspace, 16)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "workspace must be 16-byte aligned");
      const size_t wb = (size_t)need;
      if (overlap(workspace, wb, out, ob) || overlap(workspace, wb, a, span_bytes(M, K, lda, 1)) ||
          overlap(workspace, wb, w, span_bytes(N, K, ldw, 1)) ||
          overlap(workspace, wb, a_scale, (size_t)M * 4) || overlap(workspace, wb, w_scale, (size_t)N * 4) ||
          (bias && overlap(workspace, wb, bias, (size_t)N * 2)))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "workspace overlaps an input or the output");
    }
  }
  const w8a8::Epilogue epi = bias ? (gelu ? w8a8::Epilogue::kPostscaleBiasGeluBf16 : w8a8::Epilogue::kPostscaleBiasBf16)
                                  : (gelu ? w8a8::Epilogue::kPostscaleGeluBf16 : w8a8::Epilogue::kPostscaleBf16);
  return from_hip(w8a8::launch_gemm(epi, a, lda, w, ldw, a_scale, w_scale, bias, out, ldo, M, N, K,
                                    (hipStream_t)stream, run_parts, workspace),
                  name);
}

// Scratch memory of w8a8_gemm_postscale_noalloc: the split-K partial sums
// of callers that cannot allocate. Each device holds its own copy for as long
// as the library is loaded. In host code `scratch` only names the symbol; its
// device address on the current device comes from scratch_address().
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) int8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
hipError_t scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(w8a8_status_t s) {
  switch (s) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_INVALID_ARGUMENT: return "invalid argument";
    case W8A8_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (use the BF16 Linear)";
    case W8A8_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* w8a8_last_error(void) { return g_last_error.c_str(); }

const char* w8a8_version(void) { return "w8a8-gfx950 0.1"; }

int32_t w8a8_gemm_tile_channels(int64_t M, int64_t N, int64_t K, int32_t blockwise) {
  if (M < 0 || N < 128 || N % 128 || K < 128 || K % 128 || K > W8A8_MAX_K || M > kMaxRows ||
      N > kMaxRows || (blockwise != 0 && blockwise != 1))
    return -1;
  if (M == 0) return 256;
  return w8a8::use_tile160(M, N, K, w8a8::device_cu_count(), blockwise != 0) ? 160 : 256;
}

int32_t w8a8_gemm_splitk_parts(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 128) return 1;
  return w8a8::splitk_parts(M, N, K, w8a8::device_cu_count());
}

w8a8_status_t w8a8_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                              int64_t group_rows, int64_t group_cols, int8_t* q, int64_t ldq,
                              float* scale, void* stream) {
  w8a8_status_t st = check_quant_common(x, rows, cols, ldx, q, ldq, scale);
  if (st != W8A8_OK) return st;
  const bool per_row = group_rows == 1 && group_cols == cols;
  const bool g1x128 = group_rows == 1 && group_cols == 128;
  const bool g128x128 = group_rows == 128 && group_cols == 128;
  if (!(per_row || g1x128 || g128x128))
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE,
                "group (%lld, %lld) not supported: use (1, cols), (1, 128) or (128, 128)",
                (long long)group_rows, (long long)group_cols);
  if ((g1x128 || g128x128) && cols % 128)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols %% 128 != 0 for a 128-wide group");
  const int64_t n_gr = (rows + group_rows - 1) / group_rows;
  const size_t s_bytes = (size_t)(n_gr * (cols / group_cols)) * 4;
  if (overlap(q, span_bytes(rows, cols, ldq, 1), x, span_bytes(rows, cols, ldx, 2)) ||
      overlap(scale, s_bytes, x, span_bytes(rows, cols, ldx, 2)) ||
      overlap(scale, s_bytes, q, span_bytes(rows, cols, ldq, 1)))
    return fail(W8A8_ERR_INVALID_ARGUMENT, "outputs overlap each other or the input");
  if (rows == 0) return ok();
  return from_hip(w8a8::launch_quant_rows(x, rows, cols, ldx, group_rows, group_cols, q, ldq,
                                          scale, (hipStream_t)stream),
                  "w8a8_quant_rows launch");
}

w8a8_status_t w8a8_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps,
                                 int64_t rows, int64_t cols, int64_t ldx, int8_t* q, int64_t ldq,
                                 float* scale, float* inv_rms, void* stream) {
  w8a8_status_t st = check_quant_common(x, rows, cols, ldx, q, ldq, scale);
  if (st != W8A8_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f) return fail(W8A8_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (cols > w8a8::kRmsnormMaxCols)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols > %lld", (long long)w8a8::kRmsnormMaxCols);
  if (rows == 0) return ok();
  if (!gamma) return fail(W8A8_ERR_INVALID_ARGUMENT, "null gamma");
  if (!aligned(gamma, 16)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "gamma must be 16-byte aligned");
  if (inv_rms && !aligned(inv_rms, 4)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "inv_rms must be 4-byte aligned");
  const size_t xb = span_bytes(rows, cols, ldx, 2), qb = span_bytes(rows, cols, ldq, 1);
  if (overlap(q, qb, x, xb) || overlap(scale, (size_t)rows * 4, x, xb) ||
      overlap(scale, (size_t)rows * 4, q, qb) || overlap(inv_rms, (size_t)rows * 4, x, xb) ||
      overlap(inv_rms, (size_t)rows * 4, q, qb) || overlap(inv_rms, (size_t)rows * 4, scale, (size_t)rows * 4) ||
      overlap(q, qb, gamma, (size_t)cols * 2))
    return fail(W8A8_ERR_INVALID_ARGUMENT, "outputs overlap each other or an input");
  if (rows == 0) return ok();
  return from_hip(w8a8::launch_rmsnorm_quant(x, gamma, eps, rows, cols, ldx, q, ldq, scale, inv_rms,
                                             (hipStream_t)stream),
                  "w8a8_rmsnorm_quant launch");
}

w8a8_status_t w8a8_layernorm_quant(const uint16_t* x, const uint16_t* gamma,
                                   const uint16_t* beta, const uint16_t* mod_scale,
                                   const uint16_t* mod_shift, float eps, int64_t rows,
                                   int64_t cols, int64_t ldx, int8_t* q, int64_t ldq,
                                   float* out_scale, float* mean, float* rstd, void* stream) {
  w8a8_status_t st = check_quant_common(x, rows, cols, ldx, q, ldq, out_scale);
  if (st != W8A8_OK) return st;
  if (!std::isfinite(eps) || eps < 0.0f) return fail(W8A8_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (cols > w8a8::kLayernormMaxCols)
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols > %lld", (long long)w8a8::kLayernormMaxCols);
  if (rows == 0) return ok();
  const uint16_t* vecs[4] = {gamma, beta, mod_scale, mod_shift};
  for (const uint16_t* v : vecs)
    if (v && !aligned(v, 16))
      return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "gamma, beta, mod_scale and mod_shift must be 16-byte aligned");
  if ((mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4)))
    return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "mean and rstd must be 4-byte aligned");
  const size_t xb = span_bytes(rows, cols, ldx, 2), qb = span_bytes(rows, cols, ldq, 1);
  const size_t rb = (size_t)rows * 4, vb = (size_t)cols * 2;
  // outputs must not overlap each other or any input
  const void* outs[4] = {q, out_scale, mean, rstd};
  const size_t out_bytes[4] = {qb, rb, rb, rb};
  const void* ins[5] = {x, gamma, beta, mod_scale, mod_shift};
  const size_t in_bytes[5] = {xb, vb, vb, vb, vb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "outputs overlap each other or an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "outputs overlap each other or an input");
  }
  return from_hip(w8a8::launch_layernorm_quant(x, gamma, beta, mod_scale, mod_shift, eps, rows,
                                               cols, ldx, q, ldq, out_scale, mean, rstd,
                                               (hipStream_t)stream),
                  "w8a8_layernorm_quant launch");
}

w8a8_status_t w8a8_gemm_postscale(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                  const float* a_scale, const float* w_scale, uint16_t* out,
                                  int64_t ldo, int64_t M, int64_t N, int64_t K, void* stream) {
  return postscale_call("w8a8_gemm_postscale launch", a, lda, w, ldw, a_scale, w_scale, nullptr,
                        false, out, ldo, M, N, K, 1, nullptr, 0, stream);
}

w8a8_status_t w8a8_gemm_postscale_bias(const int8_t* a, int64_t lda, const int8_t* w,
                                       int64_t ldw, const float* a_scale, const float* w_scale,
                                       const uint16_t* bias, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream) {
  if (M > 0 && !bias) {
    w8a8_status_t st = check_gemm_common(a, lda, w, ldw, out, ldo, 2, M, N, K);
    return st != W8A8_OK ? st : fail(W8A8_ERR_INVALID_ARGUMENT, "null bias pointer");
  }
  return postscale_call("w8a8_gemm_postscale_bias launch", a, lda, w, ldw, a_scale, w_scale, bias,
                        false, out, ldo, M, N, K, 1, nullptr, 0, stream);
}

w8a8_status_t w8a8_gemm_postscale_gelu(const int8_t* a, int64_t lda, const int8_t* w,
                                       int64_t ldw, const float* a_scale, const float* w_scale,
                                       const uint16_t* bias, uint16_t* out, int64_t ldo,
                                       int64_t M, int64_t N, int64_t K, void* stream) {
  return postscale_call("w8a8_gemm_postscale_gelu launch", a, lda, w, ldw, a_scale, w_scale, bias,
                        true, out, ldo, M, N, K, 1, nullptr, 0, stream);
}

w8a8_status_t w8a8_gemm_postscale_ex(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                     const float* a_scale, const float* w_scale,
                                     const uint16_t* bias, int32_t flags, uint16_t* out,
                                     int64_t ldo, int64_t M, int64_t N, int64_t K, int32_t parts,
                                     void* workspace, int64_t workspace_bytes, void* stream) {
  if (flags & ~W8A8_EPILOGUE_GELU) return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", (unsigned)flags);
  return postscale_call("w8a8_gemm_postscale_ex launch", a, lda, w, ldw, a_scale, w_scale, bias,
                        (flags & W8A8_EPILOGUE_GELU) != 0, out, ldo, M, N, K, parts, workspace,
                        workspace_bytes, stream);
}

w8a8_status_t w8a8_gemm_postscale_noalloc(const int8_t* a, int64_t lda, const int8_t* w,
                                          int64_t ldw, const float* a_scale,
                                          const float* w_scale, const uint16_t* bias,
                                          int32_t flags, uint16_t* out, int64_t ldo, int64_t M,
                                          int64_t N, int64_t K, int32_t parts, void* stream) {
  if (flags & ~W8A8_EPILOGUE_GELU) return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", (unsigned)flags);
  w8a8_status_t st = check_gemm_common(a, lda, w, ldw, out, ldo, 2, M, N, K);
  if (st != W8A8_OK) return st;
  if (resolve_parts(M, N, K, parts) < 0)
    return fail(W8A8_ERR_INVALID_ARGUMENT, "parts must be 0 (library's choice) or 1..%d and at most K/128",
                w8a8::kMaxSplitParts);
  if (M == 0) return ok();
  // the library's own choice only considers splits whose partial sums fit the
  // scratch; a split the caller asks for must fit it
  const int run = parts > 0 ? parts
                            : w8a8::splitk_parts(M, N, K, w8a8::device_cu_count(), kScratchBytes);
  void* ws = nullptr;
  if (run > 1) {
    if (M * N > ((int64_t)1 << 50) || (int64_t)run * M * N * 4 > kScratchBytes)
      return fail(W8A8_ERR_INVALID_ARGUMENT,
                  "%d parts of %lld x %lld partial sums exceed the %lld-byte scratch of "
                  "w8a8_gemm_postscale_noalloc (use w8a8_gemm_postscale_ex with a workspace)",
                  run, (long long)M, (long long)N, (long long)kScratchBytes);
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return from_hip(e, "w8a8_gemm_postscale_noalloc scratch lookup");
  }
  return postscale_call("w8a8_gemm_postscale_noalloc launch", a, lda, w, ldw, a_scale, w_scale,
                        bias, (flags & W8A8_EPILOGUE_GELU) != 0, out, ldo, M, N, K, run, ws,
                        run > 1 ? kScratchBytes : 0, stream);
}

int64_t w8a8_gemm_postscale_workspace_size(int64_t M, int64_t N, int64_t K, int32_t parts) {
  if (M < 0 || N < 128 || N % 128 || K < 128 || K % 128 || K > W8A8_MAX_K || M > kMaxRows ||
      N > kMaxRows)
    return -1;
  const int resolved = resolve_parts(M, N, K, parts);
  if (resolved < 0 || (resolved > 1 && M * N > ((int64_t)1 << 50))) return -1;
  return resolved > 1 ? (int64_t)resolved * M * N * 4 : 0;
}

w8a8_status_t w8a8_gemm_blockwise(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                  const float* a_scale, const float* w_scale, uint16_t* out,
                                  int64_t ldo, int64_t M, int64_t N, int64_t K, void* stream) {
  w8a8_status_t st = check_gemm_common(a, lda, w, ldw, out, ldo, 2, M, N, K);
  if (st != W8A8_OK) return st;
  if (M == 0) return ok();
  if (!a_scale || !w_scale) return fail(W8A8_ERR_INVALID_ARGUMENT, "null scale pointer");
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "scales must be 4-byte aligned");
  const size_t ob = span_bytes(M, N, ldo, 2);
  if (overlap(out, ob, a_scale, (size_t)M * (K / 128) * 4) ||
      overlap(out, ob, w_scale, (size_t)(N / 128) * (K / 128) * 4))
    return fail(W8A8_ERR_INVALID_ARGUMENT, "output overlaps a scale");
  if (M == 0) return ok();
  return from_hip(w8a8::launch_gemm(w8a8::Epilogue::kBlockwiseBf16, a, lda, w, ldw, a_scale, w_scale, nullptr,
                                    out, ldo, M, N, K, (hipStream_t)stream),
                  "w8a8_gemm_blockwise launch");
}

w8a8_status_t w8a8_gemm_i32(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                            int32_t* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                            void* stream) {
  w8a8_status_t st = check_gemm_common(a, lda, w, ldw, out, ldo, 4, M, N, K);
  if (st != W8A8_OK) return st;
  if (M == 0) return ok();
  return from_hip(w8a8::launch_gemm(w8a8::Epilogue::kInt32, a, lda, w, ldw, nullptr, nullptr, nullptr, out,
                                    ldo, M, N, K, (hipStream_t)stream),
                  "w8a8_gemm_i32 launch");
}

}  // extern "C"
