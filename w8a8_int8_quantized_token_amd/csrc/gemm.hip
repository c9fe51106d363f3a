// INT8 x INT8 GEMM kernels for gfx950 (CDNA4 INT8 MFMA).
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", W8A8-kernel row and the paragraph under the table: the
// post-scale kernel keeps one INT32 accumulation over all of K and applies the
// activation and weight scales only in the epilogue; the original
// TurboDiffusion kernel rescales per K block (the blockwise epilogue here).
//
// out[m, n] = epilogue( sum_k a[m, k] * w[n, k] ),  a: [M, K] activation
// codes, w: [N, K] weight codes (nn.Linear layout), both K-contiguous.
//
// Design (gfx950):
//  * v_mfma_i32_16x16x64_i8. The weight tile is the MFMA "A" operand (rows =
//    output channels n) and the activation tile the "B" operand (columns =
//    tokens m), so a lane's accumulators run along n, the contiguous dimension
//    of out[M, N], and the epilogue stores 16-byte vectors.
//  * Within a wave's n range the MFMA row slots are permuted so that every
//    lane ends up holding 4*kTN consecutive output channels of one token.
//  * K advances 128 bytes per stage. Tiles move HBM/L2 -> LDS with
//    global_load_lds_dwordx4 (no VGPR staging) into a double-buffered LDS
//    ring; 16-byte chunks of each 128-byte row are XOR-swizzled so that
//    every ds_read_b128 group of 8 lanes hits 8 distinct bank groups.
//  * Tiles are numbered so that each XCD (workgroups go round-robin over the
//    8 XCDs) works on a contiguous, M-grouped range of tiles, which keeps the
//    rows it shares in its own L2.
//  * Rows past M (or N) are clamped on load and masked on store.
#include "device_common.hpp"
#include "launch.hpp"

namespace w8a8 {

constexpr int kBK = 128;        // K bytes per stage (one blockwise scale block)
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int kBN, int kBM, int kWN, int kWM>
struct GemmCfg {
  static constexpr int kWavesN = kBN / kWN;
  static constexpr int kWavesM = kBM / kWM;
  static constexpr int kWaves = kWavesN * kWavesM;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kTN = kWN / 16;          // MFMA tiles along n per wave
  static constexpr int kTM = kWM / 16;          // MFMA tiles along m per wave
  static constexpr int kStageBytes = (kBN + kBM) * kBK;
  static constexpr int kLoadsPerWave = (kBN + kBM) / 8 / kWaves;   // 1 KiB per wave-load
  static_assert((kBN + kBM) % (8 * kWaves) == 0, "tile rows must split evenly over waves");
  static_assert(kTN % 2 == 0 && kTN <= 8, "kTN in {2,4,6,8}");
  static_assert(kWN <= 128 && 128 % kWN == 0, "a wave's n range must sit inside one 128 block");
};

// Swizzle keys: which of the 8 16-byte chunks of a 128-byte LDS row holds
// logical chunk c is c ^ key(row).
template <int kTN>
__device__ __forceinline__ int key_w(int r) { return (r & 3) | (((r / (4 * kTN)) & 1) << 2); }
__device__ __forceinline__ int key_a(int r) { return r & 7; }

__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int group_m, int& tm,
                                            int& tn) {
  const int total = tiles_m * tiles_n;
  // XCD-aware renumbering: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles.
  const int xcd = b % kXcds, i = b / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + i;
  // M-grouped order inside the logical range.
  const int span = group_m * tiles_n;
  const int g = t / span;
  const int first_m = g * group_m;
  const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = t - g * span;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

template <class C, Epilogue kEpi, int kGroupM>
__global__ __launch_bounds__(C::kThreads)
void gemm_i8_kernel(const int8_t* __restrict__ a, int64_t lda, const int8_t* __restrict__ w,
                    int64_t ldw, const float* __restrict__ a_scale,
                    const float* __restrict__ w_scale, void* __restrict__ out, int64_t ldo,
                    int M, int N, int K) {
  constexpr int kBN = C::kWavesN * C::kTN * 16;
  constexpr int kBM = C::kWavesM * C::kTM * 16;
  constexpr int kTN = C::kTN, kTM = C::kTM;
  __shared__ __attribute__((aligned(1024))) int8_t lds[2 * C::kStageBytes];

  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % C::kWavesN, wm = wave / C::kWavesN;

  // ---- loader: per-lane 32-bit offsets, fixed for the whole K loop --------
  uint32_t ld_off[C::kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const int g = wave + i * C::kWaves;           // 8-row group of the [W; A] stage tile
    const int rr = 8 * g + (lane >> 3);
    const int p = lane & 7;
    if (rr < kBN) {
      const int c = p ^ key_w<kTN>(rr);
      const int row = (n0 + rr < N ? rr : N - 1 - n0);
      ld_off[i] = (uint32_t)(row * ldw + c * 16);
    } else {
      const int rb = rr - kBN;
      const int c = p ^ key_a(rb);
      const int row = (m0 + rb < M ? rb : M - 1 - m0);
      ld_off[i] = (uint32_t)(row * lda + c * 16);
    }
  }
  const int8_t* w_tile = w + (int64_t)n0 * ldw;
  const int8_t* a_tile = a + (int64_t)m0 * lda;

  auto issue_stage = [&](int kt, int buf) {
    const int8_t* wb = w_tile + (int64_t)kt * kBK;
    const int8_t* ab = a_tile + (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int g = wave + i * C::kWaves;
      const int8_t* src = (8 * g < kBN ? wb : ab) + ld_off[i];
      lds_void* dst = (lds_void*)(lds + buf * C::kStageBytes + g * 1024);
      __builtin_amdgcn_global_load_lds((const void*)src, dst, 16, 0, 0);
    }
  };

  // ---- fragment addressing -------------------------------------------------
  // W fragment of MFMA tile i, row slot ir = lane % 16 maps to wave-local
  // channel 4*kTN*(ir/4) + 4*i + ir%4; its swizzle key does not depend on i.
  const int ir = lane & 15, kq = lane >> 4;
  const int w_row0 = wn * (kTN * 16) + 4 * kTN * (ir >> 2) + (ir & 3);
  const int w_key = key_w<kTN>(w_row0);
  const int a_row0 = kBN + wm * (kTM * 16) + ir;      // stage-tile row of the A fragment
  const int a_key = key_a(a_row0 - kBN);

  v4i acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  float cacc[kEpi == Epilogue::kBlockwiseBf16 ? kTN : 1][kEpi == Epilogue::kBlockwiseBf16 ? kTM : 1][4];
  if constexpr (kEpi == Epilogue::kBlockwiseBf16) {
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) cacc[i][j][r] = 0.0f;
  }

  const int nk = K / kBK;
  const int nkb = nk;                                  // scale blocks along K
  const int n_wave = n0 + wn * (kTN * 16);             // first channel of this wave
  const int n_lane = n_wave + 4 * kTN * kq;            // first of the lane's 4*kTN channels
  const int m_lane0 = m0 + wm * (kTM * 16) + ir;       // token of MFMA column j is + 16*j

  issue_stage(0, 0);
  wait_vmcnt0();
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue_stage(kt + 1, buf ^ 1);
    const int8_t* sb = lds + buf * C::kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i fa[kTN], fb[kTM];
      const int cl = ks * 4 + kq;                       // logical 16-byte chunk
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        fa[i] = *reinterpret_cast<const v4i*>(sb + (w_row0 + 4 * i) * kBK + ((cl ^ w_key) << 4));
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        fb[j] = *reinterpret_cast<const v4i*>(sb + (a_row0 + 16 * j) * kBK + ((cl ^ a_key) << 4));
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
          if constexpr (kEpi == Epilogue::kBlockwiseBf16) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                fa[i], fb[j], ks == 0 ? v4i{0, 0, 0, 0} : acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
          }
        }
    }
    if constexpr (kEpi == Epilogue::kBlockwiseBf16) {
      // c = fmaf(fl32(acc_kb), fl32(sa[m,kb] * sw[n/128,kb]), c), ascending kb
      const int nb = (n_wave < N ? n_wave : N - 1) >> 7;   // tiles past N: any valid block
      const float swb = w_scale[(int64_t)nb * nkb + kt];
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        int m = m_lane0 + 16 * j;
        m = m < M ? m : M - 1;
        const float s = a_scale[(int64_t)m * nkb + kt] * swb;
#pragma unroll
        for (int i = 0; i < kTN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            cacc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], s, cacc[i][j][r]);
      }
    }
    wait_vmcnt0();                                   // this wave's next-stage loads landed
    __syncthreads();                                 // ... and everyone else's
  }

  // ---- epilogue ---------------------------------------------------------------
  if (n_wave >= N) return;
  if constexpr (kEpi == Epilogue::kInt32) {
    int32_t* o = reinterpret_cast<int32_t*>(out);
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int m = m_lane0 + 16 * j;
      if (m >= M) continue;
      int32_t* dst = o + (int64_t)m * ldo + n_lane;
#pragma unroll
      for (int i = 0; i < kTN; ++i)
        *reinterpret_cast<v4i*>(dst + 4 * i) = acc[i][j];
    }
  } else {
    float sw[4 * kTN];
    if constexpr (kEpi == Epilogue::kPostscaleBf16) {
#pragma unroll
      for (int e = 0; e < 4 * kTN; ++e) sw[e] = w_scale[n_lane + e];
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int m = m_lane0 + 16 * j;
      if (m >= M) continue;
      float sa = 0.0f;
      if constexpr (kEpi == Epilogue::kPostscaleBf16) sa = a_scale[m];
      uint32_t packed[2 * kTN];
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (kEpi == Epilogue::kPostscaleBf16)
            v[r] = ((float)acc[i][j][r] * sa) * sw[4 * i + r];
          else
            v[r] = cacc[i][j][r];
        }
        packed[2 * i] = pack_bf16x2(v[0], v[1]);
        packed[2 * i + 1] = pack_bf16x2(v[2], v[3]);
      }
      uint16_t* dst = o + (int64_t)m * ldo + n_lane;
#pragma unroll
      for (int h = 0; h < kTN / 2; ++h)
        *reinterpret_cast<uint4*>(dst + 8 * h) =
            make_uint4(packed[4 * h], packed[4 * h + 1], packed[4 * h + 2], packed[4 * h + 3]);
    }
  }
}

template <int kBN, int kBM, int kWN, int kWM, int kGroupM, Epilogue kEpi>
static hipError_t launch_cfg(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                             const float* a_scale, const float* w_scale, void* out, int64_t ldo,
                             int64_t M, int64_t N, int64_t K, hipStream_t st) {
  using C = GemmCfg<kBN, kBM, kWN, kWM>;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_i8_kernel<C, kEpi, kGroupM>), dim3((unsigned)tiles), dim3(C::kThreads),
                     0, st, a, lda, w, ldw, a_scale, w_scale, out, ldo, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemm(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                       const float* a_scale, const float* w_scale, void* out, int64_t ldo,
                       int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M == 0) return hipSuccess;
  switch (epi) {
    case Epilogue::kPostscaleBf16:
    case Epilogue::kInt32:
      return launch_gemm_pipelined(epi, a, lda, w, ldw, a_scale, w_scale, out, ldo, M, N, K, st);
    case Epilogue::kBlockwiseBf16:
      return launch_cfg<256, 128, 128, 64, 8, Epilogue::kBlockwiseBf16>(
          a, lda, w, ldw, a_scale, w_scale, out, ldo, M, N, K, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace w8a8
