// Persistent, software-pipelined INT8 GEMM with blockwise scales for gfx950.
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", W8A8-kernel row: the original TurboDiffusion kernel
// dequantises per K block. With 1 x 128 activation groups and 128 x 128
// weight groups, block kb of K contributes
//   acc_kb[m, n] = sum over k in [128 kb, 128 kb + 128) of a[m, k] * w[n, k]
// (exact INT32, |acc_kb| <= 127^2 * 128 < 2^24, so its fp32 conversion is
// exact too), and the output is the fp32 sum over ascending kb
//   c = fma(f32(acc_kb), f32(sa[m, kb] * sw[n / 128, kb]), c),  out = bf16(c).
//
// Structure (one workgroup of 8 waves per CU, two waves per SIMD):
//  * Block tile 256 (n) x 128 (m); each wave owns 64 x 64, held as 4 x 4
//    v_mfma_i32_16x16x64_i8 accumulators (64 registers) plus 64 fp32 running
//    sums, which leaves room for two fragment sets at two waves per SIMD.
//  * One pipeline stage is one 128-wide K block: 48 KiB of codes plus the
//    block's scales, moved into a 3-slot LDS ring by buffer loads that write
//    LDS directly. Every wave issues the same seven loads per stage (waves 0
//    and 1 bring the 128 activation scales, the others the two weight
//    scales), so each wave's vmcnt bookkeeping is the same.
//  * The rescale (a convert and an FMA per output per block: 128 VALU
//    instructions per wave per stage against 32 MFMAs) is this kernel's
//    VALU work. On gfx950 VALU instructions hide only partly behind MFMAs,
//    so it is spread thinly: the first half of the tiles is rescaled between
//    the second-K-step MFMAs of the block's own stage, the second half
//    between the first-K-step MFMAs of the next stage, just before those
//    accumulators restart at zero.
//  * Grid, tile order, LDS swizzle and row clamping follow the post-scale
//    kernel: persistent, XCD-aware, M-grouped; rows past N or M load (and
//    store) the last valid row.
#include "launch.hpp"
#include "pipeline.hpp"

namespace w8a8 {
namespace pipe {
namespace bw {

constexpr int kBN = 256, kBM = 128;   // block tile: output channels x tokens
constexpr int kBK = 128;              // one scale block of K per stage
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int kTN = 4, kTM = 4;       // 16x16 MFMA tiles per wave: 64 channels x 64 tokens
constexpr int kHalf = kTN / 2;        // tiles i < kHalf are rescaled in their own stage
constexpr int kTileBytes = (kBN + kBM) * kBK;          // 48 KiB of codes per stage
// Waves 0-3 (one per SIMD) issue all of a stage's loads; issuing them stalls
// the issuing wave, and the other wave of its SIMD keeps the MFMAs fed.
constexpr int kLoaderWaves = 4;
constexpr int kScaleArea = kLoaderWaves * 256;         // one dword wave-load per loader wave
constexpr int kSlotBytes = kTileBytes + kScaleArea;
constexpr int kLoads = kTileBytes / 1024 / kLoaderWaves;   // 1 KiB code wave-loads per loader: 12
constexpr int kStageLoads = kLoads + 1;                // plus the scale wave-load
constexpr int kRowStep = 8 * kLoaderWaves;             // rows between a loader's wave-loads
constexpr int kStoresPerTile = kTM * 2;                // 16-byte stores per wave per tile
constexpr int kGroupM = 8;
// Three slots (150 KiB of LDS) keep two stages in flight behind the one being
// consumed; two slots also work and measured about 4% slower.
constexpr int kRingSlots = 3;
static_assert(kLoads == kBN / kRowStep + kBM / kRowStep, "code rows split evenly over the loaders");

// Swizzle keys of the 128-byte LDS rows (logical 16-byte chunk c of row r at
// c ^ key(r)). A wave's weight rows are read in the permuted slot order
// 16 (s / 4) + s % 4 + 4 i, which the key keeps conflict-free.
__device__ __forceinline__ int key_w(int r) { return (r & 3) | (((r >> 4) & 1) << 2); }
__device__ __forceinline__ int key_a(int r) { return r & 7; }

template <int kSlots>
__global__ __launch_bounds__(kThreads, 1)
void gemm_i8_blockwise(const int8_t* __restrict__ a, int64_t lda, const int8_t* __restrict__ w,
                       int64_t ldw, const float* __restrict__ a_scale,
                       const float* __restrict__ w_scale, uint16_t* __restrict__ out,
                       int64_t ldo, int M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[kSlots * kSlotBytes];

  const Sched sc = make_sched(blockIdx.x, gridDim.x, tiles_m, tiles_n);
  const int nk = K / kBK;                       // stages (scale blocks) per tile
  if (sc.count == 0) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 3, wm = wave >> 2;

  // ---- loader (waves 0-3): code wave-load g fills stage rows kRowStep g + r_l
  // of the weight rows, then of the activation rows; lane -> physical chunk
  // lane % 8 (the keys ignore row bits >= 5).
  const bool loader = wave < kLoaderWaves;
  const int r_l = 8 * (wave % kLoaderWaves) + (lane >> 3);
  const int p = lane & 7;
  const int cw = (p ^ key_w(r_l)) << 4, ca = (p ^ key_a(r_l)) << 4;
  int ld_k = 0, ld_kt = 0, ld_rvn = 0, ld_rvm = 0, ld_vs = 0;
  __amdgpu_buffer_rsrc_t ld_w, ld_a, ld_s;
  auto load_tile = [&](int k) {
    int m0, n0;
    tile_mn<kBM, kBN, kGroupM>(sc, k, m0, n0);
    const int rn = (N - n0) < kBN ? (N - n0) : kBN;
    const int rm = (M - m0) < kBM ? (M - m0) : kBM;
    ld_rvn = rn - 1;
    ld_rvm = rm - 1;
    ld_w = buffer_rsrc(w + (int64_t)n0 * ldw, (uint32_t)(rn * ldw));
    ld_a = buffer_rsrc(a + (int64_t)m0 * lda, (uint32_t)(rm * lda));
    // scales: waves 0 and 1 take the activation scales of tokens 64 wave +
    // lane, the other waves the weight scales of the tile's (one or two)
    // 128-channel blocks, lane parity picking the block.
    const int ln = lane_id();
    if (wave < 2) {
      const int r = 64 * wave + ln;
      ld_s = buffer_rsrc(a_scale + (int64_t)m0 * nk, (uint32_t)(rm * nk * 4));
      ld_vs = (r < ld_rvm ? r : ld_rvm) * nk * 4;
    } else {
      const int nb = rn / 128;
      ld_s = buffer_rsrc(w_scale + (int64_t)(n0 / 128) * nk, (uint32_t)(nb * nk * 4));
      ld_vs = ((ln & 1) < nb - 1 ? (ln & 1) : nb - 1) * nk * 4;
    }
  };
  load_tile(0);
  auto issue_next = [&](int slot) {
    if (!loader) return;
    int8_t* dst = lds + slot * kSlotBytes + (wave % kLoaderWaves) * 1024;
    const int koff = ld_kt * kBK;
#pragma unroll
    for (int g = 0; g < kBN / kRowStep; ++g) {
      const int r = r_l + kRowStep * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_w, (lds_void*)(dst + g * kRowStep * kBK), 16,
                                               (r < ld_rvn ? r : ld_rvn) * (int)ldw + cw, koff,
                                               0, 0);
    }
#pragma unroll
    for (int g = 0; g < kBM / kRowStep; ++g) {
      const int r = r_l + kRowStep * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_a,
                                               (lds_void*)(dst + kBN * kBK + g * kRowStep * kBK),
                                               16, (r < ld_rvm ? r : ld_rvm) * (int)lda + ca,
                                               koff, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld_s, (lds_void*)(lds + slot * kSlotBytes + kTileBytes + wave * 256), 4, ld_vs,
        ld_kt * 4, 0, 0);
  };
  // Loader advance. It branches, so it runs at the top of a stage: placed after
  // the stage's code it would give the compiler a block past the branch into
  // which it sinks work meant to hide behind the stage's MFMAs.
  auto advance_loader = [&]() {
    if (++ld_kt == nk) {
      ld_kt = 0;
      if (++ld_k < sc.count) load_tile(ld_k);   // past the end: reloads of the last tile
    }
  };

  // ---- fragments: MFMA row slot ir of W tile i is wave-local channel
  // 16 (ir / 4) + 4 i + ir % 4, so lane (ir, kq) holds the 16 consecutive
  // channels 16 kq .. 16 kq + 15 of token ir + 16 j.
  const int ir = lane & 15, kq = lane >> 4;
  const int w_row0 = wn * 64 + 16 * (ir >> 2) + (ir & 3);
  const int a_row0 = kBN + wm * (16 * kTM) + ir;
  const int w_base = w_row0 * kBK, w_key = key_w(w_row0);
  const int a_base = a_row0 * kBK, a_key = key_a(a_row0 - kBN);
  auto read_frags = [&](v4i (&f)[kTN + kTM], int slot, int ks) {
    const int8_t* sb = lds + slot * kSlotBytes;
    const int cl = ks * 4 + kq;
    const int wo = w_base + ((cl ^ w_key) << 4), ao = a_base + ((cl ^ a_key) << 4);
#pragma unroll
    for (int i = 0; i < kTN; ++i) f[i] = *reinterpret_cast<const v4i*>(sb + wo + i * 4 * kBK);
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      f[kTN + j] = *reinterpret_cast<const v4i*>(sb + ao + j * 16 * kBK);
  };
  // scale addresses inside a slot: activation scale of token t at 4 t, weight
  // scale of the wave's 128-channel block after the 128 activation scales
  const uint32_t sa_off = kTileBytes + 4 * (wm * (16 * kTM) + ir);
  const uint32_t sw_off = kTileBytes + 512 + 4 * (wn >> 1);
  const uint32_t lds0 = lds_addr(lds);

  v4i acc[kTN][kTM];
  float c[kTN][kTM][4];
  float s_prev[kTM];             // block scales of the previous stage (0 at a tile's start)
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      acc[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) c[i][j][r] = 0.0f;
    }
#pragma unroll
  for (int j = 0; j < kTM; ++j) s_prev[j] = 0.0f;
  v4i f0[kTN + kTM], f1[kTN + kTM];

  // c += f32(acc) * s for one accumulator tile (one fma per output; with a
  // zero scale and zero sums it leaves c at +0). The empty asm uses the sums
  // where they are formed: without it the compiler sinks the whole rescale
  // past the loader's branch to the end of the stage, where it needs both
  // the old and the new accumulators and copies them.
  auto rescale = [&](int i, int j, float s) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c[i][j][r] = __builtin_fmaf((float)acc[i][j][r], s, c[i][j][r]);
    asm volatile("" : "+v"(c[i][j][0]), "+v"(c[i][j][1]), "+v"(c[i][j][2]), "+v"(c[i][j][3]));
  };

  auto epilogue = [&](int k) {
    const int el = lane_id();
    const int eir = el & 15, ekq = el >> 4;
    int m0, n0;
    tile_mn<kBM, kBN, kGroupM>(sc, k, m0, n0);
    const int n_wave = n0 + wn * 64;
    if (n_wave >= N) return;
    const int m_lane = m0 + wm * (16 * kTM) + eir;
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      // rows past M hold row M-1's values (clamped loads and scales) and store
      // them to row M-1
      int m = m_lane + 16 * j;
      m = m < M ? m : M - 1;
      uint32_t pk[2 * kTN];
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        pk[2 * i] = pack_bf16x2(c[i][j][0], c[i][j][1]);
        pk[2 * i + 1] = pack_bf16x2(c[i][j][2], c[i][j][3]);
      }
      uint16_t* dst = out + (int64_t)m * ldo + n_wave + 16 * ekq;
      *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
  };

  // Stores are counted at the next tile's first barrier only when every wave
  // stores (N a multiple of 256); otherwise that wait covers them too.
  const int stores_per_tile = (N % kBN == 0) ? kStoresPerTile : 0;
  int pending_stores = 0;

  // ---- prologue: the first kSlots stages in flight; stage 0's K step 0
  // fragments ----
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    if (i > 0) advance_loader();
    issue_next(i);
  }
  if (loader) wait_vmcnt<kStageLoads * (kSlots - 1)>();   // stage 0 landed
  lds_barrier();
  read_frags(f0, 0, 0);

  int slot = 0;
  for (int k = 0; k < sc.count; ++k) {
    for (int kt = 0; kt < nk; ++kt) {
      const int next = slot + 1 == kSlots ? 0 : slot + 1;
      const uint32_t sl = lds0 + slot * kSlotBytes;
      advance_loader();                    // to stage s + kSlots
      // ---- K step 0: accumulators restart at zero; the previous block's
      // second-half rescale goes first, tile by tile, between the MFMAs.
      float sa[kTM], swv;
#pragma unroll
      for (int j = 0; j < kTM; ++j) sa[j] = lds_read_f1(sl + sa_off + 4 * 16 * j);
      swv = lds_read_f1(sl + sw_off);
      read_frags(f1, slot, 1);
#pragma unroll
      for (int i = 0; i < kHalf; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0[i], f0[kTN + j], v4i{0, 0, 0, 0},
                                                             0, 0, 0);
#pragma unroll
      for (int i = kHalf; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
          rescale(i, j, s_prev[j]);
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0[i], f0[kTN + j], v4i{0, 0, 0, 0},
                                                             0, 0, 0);
        }
#pragma unroll
      for (int q = 0; q < kHalf * kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, (kTN - kHalf) * kTM, 0);
      __builtin_amdgcn_sched_barrier(0);
      // this wave's reads of slot `slot` are done (the wait names the scale
      // registers so no use of them moves above it); stage s+1 has landed
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(swv)
                   :
                   : "memory");
      // (the loads of the kSlots - 2 stages after it and the previous tile's
      // stores may still be in flight)
      if (loader) {
        if (pending_stores) wait_vmcnt<kStageLoads * (kSlots - 2) + kStoresPerTile>();
        else wait_vmcnt<kStageLoads * (kSlots - 2)>();
      }
      lds_barrier();                       // ... for every wave; slot `slot` is free
      __builtin_amdgcn_sched_barrier(0);
      pending_stores = 0;
      float s_cur[kTM];
#pragma unroll
      for (int j = 0; j < kTM; ++j) s_cur[j] = sa[j] * swv;
      // ---- K step 1, the refill of this slot, the next stage's first
      // fragments, and this block's first-half rescale after its MFMAs.
      issue_next(slot);                    // stage s + kSlots
      read_frags(f0, next, 0);
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f1[i], f1[kTN + j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < kHalf; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) rescale(i, j, s_cur[j]);
#pragma unroll
      for (int q = 0; q < kHalf * kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 2, 0);
      }
#pragma unroll
      for (int q = 0; q < (kTN - kHalf) * kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kTM; ++j) s_prev[j] = s_cur[j];
      slot = next;
    }
    // the tile's last block: second-half rescale, then the output
#pragma unroll
    for (int i = kHalf; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) rescale(i, j, s_prev[j]);
    epilogue(k);
    pending_stores = stores_per_tile;
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) c[i][j][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < kTM; ++j) s_prev[j] = 0.0f;
  }
  // LDS DMA still in flight must land before the workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace bw
}  // namespace pipe

hipError_t launch_gemm_blockwise(const int8_t* a, int64_t lda, const int8_t* w, int64_t ldw,
                                 const float* a_scale, const float* w_scale, uint16_t* out,
                                 int64_t ldo, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int tiles_m = (int)((M + pipe::bw::kBM - 1) / pipe::bw::kBM);
  const int tiles_n = (int)((N + pipe::bw::kBN - 1) / pipe::bw::kBN);
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  const int cus = device_cu_count();
  const int grid = (int)(tiles < cus ? tiles : cus);
  hipLaunchKernelGGL(pipe::bw::gemm_i8_blockwise<pipe::bw::kRingSlots>, dim3(grid), dim3(pipe::bw::kThreads), 0, st, a,
                     lda, w, ldw, a_scale, w_scale, out, ldo, (int)M, (int)N, (int)K, tiles_m,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace w8a8
