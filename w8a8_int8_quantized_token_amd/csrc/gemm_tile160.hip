// INT8 GEMM with 128-token x 160-channel tiles, for GEMMs whose 256 x 256
// tiles would leave most compute units idle (about a thousand tokens): at
// M = 1000 and N = 5120 the 256 x 256 tiling makes 80 tiles for 256 compute
// units, this one 8 x 32 = 256.
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion": the post-scale kernel keeps one INT32 accumulation over all
// of K and applies the activation and weight scales in the epilogue (the
// paragraph under the table); the original kernel rescales per 128-wide K
// block (W8A8-kernel row). Both epilogues run here with the same fp32 steps,
// in the same order, as the 256 x 256 kernels, so the outputs are identical.
//
// Structure (one workgroup of 8 waves per tile, one tile per workgroup):
//  * K streams in 128-byte stages (160 weight rows + 128 activation rows,
//    36 KiB) through a 3-slot LDS ring filled by buffer loads that write LDS
//    directly; waves 0-3 issue all of a stage's loads (one loader wave per
//    SIMD: issuing the loads stalls the issuing wave, and the other wave of
//    its SIMD keeps the MFMAs fed). Past the last stage the loaders reload a
//    valid stage into slots nothing reads, so every stage waits on the same
//    load count.
//  * Post-scale (gemm_i8_t160_postscale): the two waves of a SIMD share 64
//    tokens x 80 channels and take alternate 64-byte K steps, each into its
//    own INT32 sums, added exactly at the end.
//  * Blockwise (gemm_i8_t160_blockwise): each wave owns 32 tokens x 80
//    channels over both K steps, with two accumulator sets: stage s
//    accumulates its block into one while the previous block's sums are
//    rescaled into the fp32 sums between the MFMAs.
//  * W rows are the MFMA A operand, tokens the B operand
//    (v_mfma_i32_16x16x64_i8). Rows past M or N load the last valid row;
//    their results are not stored.
//  * The workgroup -> tile map is XCD-aware: workgroup b runs on XCD b % 8,
//    and each XCD takes a contiguous range of tiles (all token tiles of a few
//    channel tiles), so the weight rows its tiles share stay in its L2.
#include <type_traits>

#include "launch.hpp"
#include "pipeline.hpp"

namespace w8a8 {
namespace pipe {
namespace t160 {

constexpr int kBM = 128, kBN = 160;    // tile: tokens x output channels
constexpr int kBK = 128;               // K bytes per stage (two 64-byte MFMA K steps)
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int kTN = 5, kTM = 2;        // 16x16 MFMA tiles per wave: 80 channels x 32 tokens
constexpr int kRows = kBN + kBM;       // LDS rows per stage: weight rows, then activation rows
constexpr int kCodeBytes = kRows * kBK;             // 36 KiB
constexpr int kLoaderWaves = 4;
constexpr int kWLoads = kBN / (8 * kLoaderWaves);   // weight wave-loads per loader: 5
constexpr int kALoads = kBM / (8 * kLoaderWaves);   // activation wave-loads per loader: 4
constexpr int kScaleArea = kLoaderWaves * 256;      // blockwise: one dword wave-load per loader
constexpr int kSlots = 3;             // four measured no faster
constexpr int kGroupM = 8;                           // token tiles per tile-order group
static_assert(kWLoads * 8 * kLoaderWaves == kBN && kALoads * 8 * kLoaderWaves == kBM, "rows");

// 128-byte LDS rows hold 8 chunks of 16 bytes; logical chunk c of LDS row r
// sits at c ^ (r & 7). Fragment reads take 16 consecutive rows at one logical
// chunk, which this key keeps free of bank conflicts.
__device__ __forceinline__ int row_key(int r) { return r & 7; }

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// The blockwise-scaled GEMM: per 128-wide K block kb, in ascending order,
// c = fmaf(fl32(block sum), fl32(a_scale[m, kb] * w_scale[n / 128, kb]), c);
// out = bf16(c).
__global__ __launch_bounds__(kThreads, 1)
void gemm_i8_t160_blockwise(const int8_t* __restrict__ a, int64_t lda,
                            const int8_t* __restrict__ w, int64_t ldw,
                            const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                            uint16_t* __restrict__ out, int64_t ldo, int M, int N, int K,
                            int tiles_m, int tiles_n) {
  constexpr int kSlotBytes = kCodeBytes + kScaleArea;
  constexpr int kStageLoads = kWLoads + kALoads + 1;
  __shared__ __attribute__((aligned(1024))) int8_t lds[kSlots * kSlotBytes];

  // this workgroup's tile
  const Sched sc = make_sched(blockIdx.x, gridDim.x, tiles_m, tiles_n);
  if (sc.count == 0) return;
  int m0, n0;
  tile_mn<kBM, kBN, kGroupM>(sc, 0, m0, n0);
  const int nk = K / kBK;
  const int rn = (N - n0) < kBN ? (N - n0) : kBN;    // valid rows of the tile
  const int rm = (M - m0) < kBM ? (M - m0) : kBM;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const bool loader = wave < kLoaderWaves;

  // ---- loader (waves 0-3): weight wave-load g fills LDS rows 8 (v + 4 g) +
  // lane / 8, activation wave-load g rows kBN + 8 (v + 4 g) + lane / 8; lane ->
  // physical chunk lane % 8, logical chunk (lane % 8) ^ (lane / 8).
  const int v = wave % kLoaderWaves;
  const int lr = 8 * v + (lane >> 3);                   // row of wave-load 0
  const int chunk = ((lane & 7) ^ row_key(lane >> 3)) << 4;
  const __amdgpu_buffer_rsrc_t ld_w = buffer_rsrc(w + (int64_t)n0 * ldw, (uint32_t)(rn * ldw));
  const __amdgpu_buffer_rsrc_t ld_a = buffer_rsrc(a + (int64_t)m0 * lda, (uint32_t)(rm * lda));
  // a stage's scales: loaders 0 and 1 bring the activation scales of tokens
  // 64 v + lane, loaders 2 and 3 the weight scales of the tile's (at most two)
  // 128-channel blocks, lane parity picking the block (a 160-channel window
  // starting at a multiple of 160 spans at most two 128-channel blocks)
  __amdgpu_buffer_rsrc_t ld_s;
  int s_voff = 0;
  if (v < 2) {
    const int t = 64 * v + lane;
    ld_s = buffer_rsrc(a_scale + (int64_t)m0 * nk, (uint32_t)(rm * nk * 4));
    s_voff = (t < rm - 1 ? t : rm - 1) * nk * 4;
  } else {
    const int b0 = n0 / 128, nb = N / 128;
    const int b = b0 + (lane & 1) < nb - 1 ? b0 + (lane & 1) : nb - 1;
    ld_s = buffer_rsrc(w_scale, (uint32_t)(nb * nk * 4));
    s_voff = b * nk * 4;
  }
  auto issue = [&](int stage, int slot) {
    if (!loader) return;
    const int ks = stage < nk ? stage : nk - 1;        // past the end: reload the last stage
    const int koff = ks * kBK;
    int8_t* dst = lds + slot * kSlotBytes + v * 1024;
#pragma unroll
    for (int g = 0; g < kWLoads; ++g) {
      const int r = lr + 32 * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_w, (lds_void*)(dst + g * 4096), 16,
                                               (r < rn - 1 ? r : rn - 1) * (int)ldw + chunk, koff,
                                               0, 0);
    }
#pragma unroll
    for (int g = 0; g < kALoads; ++g) {
      const int r = lr + 32 * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_a, (lds_void*)(dst + kBN * kBK + g * 4096), 16,
                                               (r < rm - 1 ? r : rm - 1) * (int)lda + chunk, koff,
                                               0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ld_s, (lds_void*)(lds + slot * kSlotBytes + kCodeBytes + v * 256), 4, s_voff, ks * 4, 0,
        0);
  };

  const int ir = lane & 15, kq = lane >> 4;
  const int n_lane = n0 + wn * 80 + 4 * kq;            // + 16 i + e
  const int m_lane = m0 + wm * 32 + ir;                // + 16 j

  // ---- fragments: W tile i = LDS rows 80 wn + 16 i + ir, activation tile j =
  // rows kBN + 32 wm + 16 j + ir; lane (ir, kq) holds 16 K bytes at logical
  // chunk 4 ks + kq of its row.
  const int w_row = wn * 80 + ir, a_row = kBN + wm * 32 + ir;
  const int key = row_key(ir);                          // the row bases are multiples of 16
  auto read_frags = [&](v4i (&f)[kTN + kTM], int slot, int ks) {
    const int8_t* sb = lds + slot * kSlotBytes + (((ks * 4 + kq) ^ key) << 4);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
      f[i] = *reinterpret_cast<const v4i*>(sb + (w_row + 16 * i) * kBK);
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      f[kTN + j] = *reinterpret_cast<const v4i*>(sb + (a_row + 16 * j) * kBK);
  };

  v4i acc[2][kTN][kTM];            // two sets of block sums, alternating per stage
  float c[kTN][kTM][4];            // the fp32 sums
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        acc[h][i][j] = v4i{0, 0, 0, 0};
        c[i][j][0] = c[i][j][1] = c[i][j][2] = c[i][j][3] = 0.0f;
      }
  v4i f0[kTN + kTM], f1[kTN + kTM];

  // scale addresses inside a slot (activation scale of token t at
  // 4 t; the weight scales of blocks n0 / 128 and n0 / 128 + 1 at 512 and 516)
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t sa_off = kCodeBytes + 4 * (wm * 32 + ir);
  int w_blk[kTN];                  // 0 or 1: the block of channels n_lane + 16 i
#pragma unroll
  for (int i = 0; i < kTN; ++i) w_blk[i] = (n_lane + 16 * i) / 128 - n0 / 128;
  float s_prev[kTN][kTM];          // the previous stage's block scales
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) s_prev[i][j] = 0.0f;

  // ---- prologue: stages 0 .. kSlots-1 in flight, stage 0's K step 0 read ----
#pragma unroll
  for (int i = 0; i < kSlots; ++i) issue(i, i);
  if (loader) wait_vmcnt<kStageLoads * (kSlots - 1)>();
  lds_barrier();
  read_frags(f0, 0, 0);

  // One stage; H (compile-time, the stage's parity) picks the accumulator
  // set, so both sets stay in registers.
  int slot = 0;
  auto stage = [&](auto hc, int s) {
    constexpr int h = decltype(hc)::value;
    const int next = slot + 1 == kSlots ? 0 : slot + 1;
    float s_cur[kTN][kTM];
    {
      // this block's scales: 2 activation scales, the tile's 2 weight scales
      const uint32_t sl = lds0 + slot * kSlotBytes;
      float sa0 = lds_read_f1(sl + sa_off), sa1 = lds_read_f1(sl + sa_off + 64);
      float sw0 = lds_read_f1(sl + kCodeBytes + 512), sw1 = lds_read_f1(sl + kCodeBytes + 516);
      read_frags(f1, slot, 1);
      // K step 0 restarts set h at zero; set h ^ 1 (the previous block) is
      // rescaled between the MFMAs
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            c[i][j][r] = __builtin_fmaf((float)acc[h ^ 1][i][j][r], s_prev[i][j], c[i][j][r]);
          acc[h][i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0[i], f0[kTN + j],
                                                               v4i{0, 0, 0, 0}, 0, 0, 0);
        }
#pragma unroll
      for (int q = 0; q < kTN * kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sa0), "+v"(sa1), "+v"(sw0), "+v"(sw1) : : "memory");
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        const float swi = w_blk[i] ? sw1 : sw0;
        s_cur[i][0] = sa0 * swi;
        s_cur[i][1] = sa1 * swi;
      }
    }
    // every wave is done with slot `slot`, and stage s + 1 has landed
    if (loader) wait_vmcnt<kStageLoads * (kSlots - 2)>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + kSlots, slot);
    read_frags(f0, next, 0);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        acc[h][i][j] =
            __builtin_amdgcn_mfma_i32_16x16x64_i8(f1[i], f1[kTN + j], acc[h][i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < kTN + kTM; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 3, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) s_prev[i][j] = s_cur[i][j];
    slot = next;
  };
  // the last block's sums into the fp32 sums (set H)
  auto finish = [&](auto hc) {
    constexpr int h = decltype(hc)::value;
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          c[i][j][r] = __builtin_fmaf((float)acc[h][i][j][r], s_prev[i][j], c[i][j][r]);
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    stage(H0{}, s);
    stage(H1{}, s + 1);
  }
  if (s < nk) stage(H0{}, s);
  if ((nk - 1) & 1) finish(H1{});
  else finish(H0{});
  // the reloads past the end must land before the workgroup's LDS is released
  wait_vmcnt<0>();

  // ---- epilogue: lane (ir, kq) holds channels n_lane + 16 i + [0, 4) of token
  // m_lane + 16 j; each such run is one 8-byte store. The stores are ordinary
  // ones: a line's five 32-byte pieces come from one wave and are merged in
  // the L2 (non-temporal stores sent each piece to memory on its own and made
  // the epilogue 2.5 times longer).
#pragma unroll
  for (int j = 0; j < kTM; ++j) {
    const int m = m_lane + 16 * j;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n_lane + 16 * i;
      const float* vv = c[i][j];
      if (m < M && n < N)
        *reinterpret_cast<v2u*>(out + (int64_t)m * ldo + n) =
            v2u{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
    }
  }
}

// Post-scale variant with the K steps split between the two waves of a
// SIMD: wave pair q (waves q and q + 4) owns 64 tokens x 80 channels (4 x 5
// MFMA tiles); wave q computes the first 64-byte K step of every stage and
// wave q + 4 the second, each into its own INT32 sums. Each wave then reads
// 9 fragments per 20 MFMAs instead of 7 per 10. At the end the two partial
// sums of every output are added (INT32, exact) through LDS, each wave of the
// pair finishing half of the tokens.
template <Epilogue kEpi>
__global__ __launch_bounds__(kThreads, 1)
void gemm_i8_t160_postscale(const int8_t* __restrict__ a, int64_t lda,
                            const int8_t* __restrict__ w, int64_t ldw,
                            const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                            const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                            int64_t ldo, int M, int N, int K, int tiles_m, int tiles_n) {
  constexpr bool kBias = epilogue_has_bias(kEpi);
  constexpr bool kGelu = epilogue_has_gelu(kEpi);
  constexpr int kSlotBytes = kCodeBytes;
  constexpr int kStageLoads = kWLoads + kALoads;
  constexpr int kPM = 4;               // 16-token MFMA tiles per wave: 64 tokens
  constexpr int kXBytes = 4 * 2 * kTN * kWave * 16;   // one direction of the exchange: 40 KiB
  static_assert(2 * kXBytes <= kSlots * kSlotBytes, "the exchange reuses the ring");
  __shared__ __attribute__((aligned(1024))) int8_t lds[kSlots * kSlotBytes];

  const Sched sc = make_sched(blockIdx.x, gridDim.x, tiles_m, tiles_n);
  if (sc.count == 0) return;
  int m0, n0;
  tile_mn<kBM, kBN, kGroupM>(sc, 0, m0, n0);
  const int nk = K / kBK;
  const int rn = (N - n0) < kBN ? (N - n0) : kBN;
  const int rm = (M - m0) < kBM ? (M - m0) : kBM;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pq = wave & 3, hk = wave >> 2;             // pair (SIMD) and K step
  const int wm2 = pq >> 1, wn2 = pq & 1;
  const bool loader = wave < kLoaderWaves;

  // ---- loader (waves 0-3), as in gemm_i8_t160_blockwise ----
  const int v = wave % kLoaderWaves;
  const int lr = 8 * v + (lane >> 3);
  const int chunk = ((lane & 7) ^ row_key(lane >> 3)) << 4;
  const __amdgpu_buffer_rsrc_t ld_w = buffer_rsrc(w + (int64_t)n0 * ldw, (uint32_t)(rn * ldw));
  const __amdgpu_buffer_rsrc_t ld_a = buffer_rsrc(a + (int64_t)m0 * lda, (uint32_t)(rm * lda));
  auto issue = [&](int stage, int slot) {
    if (!loader) return;
    const int koff = (stage < nk ? stage : nk - 1) * kBK;   // past the end: reload the last stage
    int8_t* dst = lds + slot * kSlotBytes + v * 1024;
#pragma unroll
    for (int g = 0; g < kWLoads; ++g) {
      const int r = lr + 32 * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_w, (lds_void*)(dst + g * 4096), 16,
                                               (r < rn - 1 ? r : rn - 1) * (int)ldw + chunk, koff,
                                               0, 0);
    }
#pragma unroll
    for (int g = 0; g < kALoads; ++g) {
      const int r = lr + 32 * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_a, (lds_void*)(dst + kBN * kBK + g * 4096), 16,
                                               (r < rm - 1 ? r : rm - 1) * (int)lda + chunk, koff,
                                               0, 0);
    }
  };

  // ---- epilogue operands (the oldest loads): this wave finishes tiles
  // j = 2 hk, 2 hk + 1 of the pair's 4 token tiles
  const int ir = lane & 15, kq = lane >> 4;
  const int n_lane = n0 + wn2 * 80 + 4 * kq;           // + 16 i + e
  const int m_lane = m0 + wm2 * 64 + 32 * hk + ir;     // + 16 jj
  float e_sa[2], e_sw[kTN][4];
  uint32_t e_b[kTN][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int m = m_lane + 16 * jj;
    e_sa[jj] = a_scale[m < M ? m : M - 1];
  }
#pragma unroll
  for (int i = 0; i < kTN; ++i) {
    const int n = n_lane + 16 * i;
    const int nc = n < N ? n : N - 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) e_sw[i][e] = w_scale[nc + e];
    if constexpr (kBias) {
      const uint2 b2 = *reinterpret_cast<const uint2*>(bias + nc);
      e_b[i][0] = b2.x;
      e_b[i][1] = b2.y;
    }
  }

  // ---- fragments of this wave's K step: W tile i = LDS rows 80 wn2 + 16 i +
  // ir, token tile j = rows kBN + 64 wm2 + 16 j + ir, logical chunk 4 hk + kq
  const int w_row = wn2 * 80 + ir, a_row = kBN + wm2 * 64 + ir;
  const int coff = ((hk * 4 + kq) ^ row_key(ir)) << 4;
  auto read_frags = [&](v4i (&f)[kTN + kPM], int slot) {
    const int8_t* sb = lds + slot * kSlotBytes + coff;
#pragma unroll
    for (int i = 0; i < kTN; ++i)
      f[i] = *reinterpret_cast<const v4i*>(sb + (w_row + 16 * i) * kBK);
#pragma unroll
    for (int j = 0; j < kPM; ++j)
      f[kTN + j] = *reinterpret_cast<const v4i*>(sb + (a_row + 16 * j) * kBK);
  };

  v4i acc[kTN][kPM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kPM; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  v4i fa[kTN + kPM], fb[kTN + kPM];

  // ---- prologue: stages 0 .. kSlots-1 in flight; stage 0 landed and read ----
#pragma unroll
  for (int i = 0; i < kSlots; ++i) issue(i, i);
  if (loader) wait_vmcnt<kStageLoads * (kSlots - 1)>();
  lds_barrier();
  read_frags(fa, 0);

  // Stage s: at its barrier stage s + 1 has landed and every wave has read
  // stage s (its fragments are in registers), so slot s % kSlots is refilled
  // with stage s + kSlots while this stage's MFMAs run and stage s + 1's
  // fragments are read.
  int slot = 0;
  auto stage = [&](v4i (&fc)[kTN + kPM], v4i (&fn)[kTN + kPM], int s) {
    const int next = slot + 1 == kSlots ? 0 : slot + 1;
    wait_lgkmcnt0();
    if (loader) wait_vmcnt<kStageLoads * (kSlots - 2)>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + kSlots, slot);
    read_frags(fn, next);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kPM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fc[i], fc[kTN + j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < kTN + kPM; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    slot = next;
  };
  int s = 0;
  for (; s + 1 < nk; s += 2) {
    stage(fa, fb, s);
    stage(fb, fa, s + 1);
  }
  if (s < nk) stage(fa, fb, s);

  // ---- the two partial sums: every wave leaves the tiles its partner
  // finishes in LDS, then adds the partner's partials of its own tiles ----
  wait_vmcnt<0>();                 // the reloads past the end have landed
  wait_lgkmcnt0();
  lds_barrier();                   // ... and no wave reads the ring any more
  auto xslot = [&](int dir, int jj, int i) {
    return reinterpret_cast<v4i*>(lds + dir * kXBytes) + ((pq * 2 + jj) * kTN + i) * kWave + lane;
  };
  // (the halves are picked by a wave-uniform branch: indexing the sums with
  // hk itself would move them to scratch memory)
  v4i mine[kTN][2], theirs[kTN][2];
  if (hk) {
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        mine[i][jj] = acc[i][2 + jj];
        theirs[i][jj] = acc[i][jj];
      }
  } else {
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        mine[i][jj] = acc[i][jj];
        theirs[i][jj] = acc[i][2 + jj];
      }
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < kTN; ++i) *xslot(hk, jj, i) = theirs[i][jj];
  lds_barrier();
  v4i tot[kTN][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < kTN; ++i) tot[i][jj] = mine[i][jj] + *xslot(1 - hk, jj, i);

  // ---- epilogue: lane (ir, kq) holds channels n_lane + 16 i + [0, 4) of token
  // m_lane + 16 jj; each such run is one 8-byte store (ordinary stores, as in
  // gemm_i8_t160_blockwise)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int m = m_lane + 16 * jj;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n_lane + 16 * i;
      float vv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[r] = ((float)tot[i][jj][r] * e_sa[jj]) * e_sw[i][r];
      if constexpr (kBias) {
        vv[0] = vv[0] + bf16_lo(e_b[i][0]);
        vv[1] = vv[1] + bf16_hi(e_b[i][0]);
        vv[2] = vv[2] + bf16_lo(e_b[i][1]);
        vv[3] = vv[3] + bf16_hi(e_b[i][1]);
      }
      if constexpr (kGelu) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = gelu_erf(round_bf16(vv[r]));
      }
      if (m < M && n < N)
        *reinterpret_cast<v2u*>(out + (int64_t)m * ldo + n) =
            v2u{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
    }
  }
}

}  // namespace t160
}  // namespace pipe

int tile160_tiles(int64_t M, int64_t N) {
  return (int)(((M + pipe::t160::kBM - 1) / pipe::t160::kBM) *
               ((N + pipe::t160::kBN - 1) / pipe::t160::kBN));
}

hipError_t launch_gemm_tile160(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w,
                               int64_t ldw, const float* a_scale, const float* w_scale,
                               const uint16_t* bias, uint16_t* out, int64_t ldo, int64_t M,
                               int64_t N, int64_t K, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int tiles_m = (int)((M + pipe::t160::kBM - 1) / pipe::t160::kBM);
  const int tiles_n = (int)((N + pipe::t160::kBN - 1) / pipe::t160::kBN);
  const dim3 grid(tiles_m * tiles_n), block(pipe::t160::kThreads);
  if (epi == Epilogue::kBlockwiseBf16) {
    hipLaunchKernelGGL(pipe::t160::gemm_i8_t160_blockwise, grid, block, 0, st, a, lda, w, ldw,
                       a_scale, w_scale, out, ldo, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    return hipGetLastError();
  }
#define W8A8_T160_LAUNCH(E)                                                                   \
  hipLaunchKernelGGL((pipe::t160::gemm_i8_t160_postscale<E>), grid, block, 0, st, a, lda, w, \
                     ldw, a_scale, w_scale, bias, out, ldo, (int)M, (int)N, (int)K, tiles_m,   \
                     tiles_n)
  switch (epi) {
    case Epilogue::kPostscaleBf16: W8A8_T160_LAUNCH(Epilogue::kPostscaleBf16); break;
    case Epilogue::kPostscaleBiasBf16: W8A8_T160_LAUNCH(Epilogue::kPostscaleBiasBf16); break;
    case Epilogue::kPostscaleGeluBf16: W8A8_T160_LAUNCH(Epilogue::kPostscaleGeluBf16); break;
    case Epilogue::kPostscaleBiasGeluBf16:
      W8A8_T160_LAUNCH(Epilogue::kPostscaleBiasGeluBf16);
      break;
    default: return hipErrorInvalidValue;
  }
#undef W8A8_T160_LAUNCH
  return hipGetLastError();
}

}  // namespace w8a8
