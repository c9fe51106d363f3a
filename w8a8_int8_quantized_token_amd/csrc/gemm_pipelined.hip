// Persistent, software-pipelined INT8 GEMM for gfx950 (post-scale and INT32
// epilogues).
//
// "TurboDiffusion Integration Notes", section "Differences From
// TurboDiffusion", paragraph under the table: one INT32 accumulation runs over
// all of K; the activation and weight scales are applied in the epilogue.
//
// out[m, n] = epilogue( sum_k a[m, k] * w[n, k] ), a [M, K] and w [N, K] INT8,
// both K-contiguous.
//
// Structure (one workgroup of 8 waves per CU, two waves per SIMD):
//  * Block tile 256 (n) x 256 (m); each wave owns 128 x 64, held as 8 x 4
//    v_mfma_i32_16x16x64_i8 accumulators (128 registers).
//  * K is streamed in 128-byte stages through a 2-slot LDS ring (64 KiB per
//    slot) filled by buffer loads that write LDS directly (no register
//    staging); a load's address is a descriptor base plus a 32-bit lane
//    offset plus the stage's K offset in an SGPR.
//  * Fragments are read one 64-byte K step ahead into a second register set,
//    so every MFMA finds its operands ready. The single stage barrier sits
//    between the two K steps of a stage: after it, the next stage's first
//    fragments are read and the slot just drained is refilled, both hidden
//    behind the second K step's MFMAs.
//  * The grid is persistent (one workgroup per CU) and walks its tiles back
//    to back: the next tile's first stages are in flight during an epilogue.
//    Workgroup b sits on XCD b % 8; each XCD owns a contiguous, M-grouped
//    range of tiles so shared rows stay in that XCD's L2.
//  * Weight rows are the MFMA "A" operand with permuted row slots: the four
//    lanes of a token hold 32 consecutive output channels in each of two
//    packed values (16-byte pieces scattered over more lines cost the
//    epilogue about 40% more time), and a swap between lanes 8 apart pairs
//    them so that one store instruction writes 8 tokens x 128 contiguous
//    bytes, whole lines. The stores are non-temporal: with whole lines they
//    write exactly the output's bytes (half lines cost a third more).
//  * With M and N of at least one tile, the last tile row and column are
//    moved back to end at M and N (they overlap their neighbours, whose
//    rows they recompute and store again with identical values), so every
//    load is in range and its offset is a lane constant plus a scalar. Below
//    that, rows past M or N load the last valid row instead.
//  * LDS rows are XOR-swizzled in 16-byte chunks. A ds_read_b128 is served
//    16 lanes at a time and is conflict-free when those lanes hit 16
//    distinct 16-byte slots of the 256-byte bank line; the keys below give
//    every such lane group of the fragment reads distinct slots.
#include <atomic>

#include "launch.hpp"
#include "pipeline.hpp"

namespace w8a8 {
namespace pipe {

constexpr int kBN = 256, kBM = 256;   // block tile: output channels x tokens
constexpr int kBK = 128;              // K bytes per stage (two 64-byte MFMA K steps)
constexpr int kSlots = 2;             // LDS ring of stages
constexpr int kSlotBytes = (kBN + kBM) * kBK;   // 64 KiB
constexpr int kWaves = 8, kThreads = kWaves * kWave;
constexpr int kTN = 8, kTM = 4;       // 16x16 MFMA tiles per wave: 128 channels x 64 tokens
constexpr int kLoaderWaves = 4;       // waves that issue the stage refills (one per SIMD)
constexpr int kLoads = (kBN + kBM) * kBK / 1024 / kLoaderWaves;   // 1 KiB wave-loads per loader wave
constexpr int kStoresPerTile = kTM * 4;                       // 16-byte stores per wave per tile
constexpr int kScaleBytes = (kBN + kBM) * 4;   // one tile's scales
constexpr int kBiasBytes = kWaves * 256;       // one dword wave-load per wave (the tile's
                                               // 256 BF16 biases fill the first 512 bytes)
constexpr int kScaleBufs = 3;                  // tile k's scales sit in buffer k % 3
constexpr int kGroupM = 4;

// GELU of a BF16 value y (to BF16), by ranges of its exponent field e:
//  * e <= 117 (|y| < 2^-9): GELU(y) rounds to the BF16 rounding of y/2
//    (GELU(y) / (y/2) - 1 is about y * sqrt(2/pi), below half a BF16 unit
//    there; checked for every such y), and y * 0.5f is exact in fp32;
//  * e in [118, 130], either sign: a 3328-entry table (6.5 KiB of LDS) built
//    at kernel start with the erfc formula, which is correctly rounded for
//    every BF16 input there: entry (bits & 0x7FFF) - (118 << 7), plus 1664
//    for negative y;
//  * e >= 131 (|y| >= 16): y for positive y (GELU(y) rounds to y from
//    2.78125 on), -0 for negative y (from -13.5625 on); +inf gives +inf,
//    -inf and NaN give NaN, as y/2 * erfc(-y / sqrt(2)) does.
// The values are handled in pairs, packed as they are stored (the first in
// the low 16 bits), with 16-bit packed integer arithmetic: a clamped table
// offset is formed for both values and both entries are read into the two
// halves of one register; the selection then picks the entry, y/2 or the far
// value per half. The last entry of the negative half is GELU(-15.9375) = -0,
// so a finite negative y past the table takes its clamped entry as well.
constexpr int kGeluFirstExp = 118;
constexpr int kGeluHalf = 13 * 128;            // entries per sign: e = 118 .. 130
constexpr int kGeluTable = 2 * kGeluHalf;      // entries (uint16)
constexpr uint32_t kGeluLow = (uint32_t)kGeluFirstExp << 7;

__device__ __forceinline__ uint16_t gelu_table_entry(int i) {
  const uint32_t neg = i >= kGeluHalf ? 1u : 0u;
  const uint32_t mag = kGeluLow + (uint32_t)(neg ? i - kGeluHalf : i);
  const float y = __uint_as_float(((neg << 15) | mag) << 16);
  return (uint16_t)(pack_bf16x2(gelu_erf(y), 0.0f) & 0xFFFFu);
}

// Per 16-bit half of a packed BF16 pair p (magnitude bits a, sign s):
//  * i2 = 2 (a - low) mod 2^16, computed as 2 p - 2 low (the sign bit
//    shifts out): below the table it wraps to 0x8A00 or more, above it stays
//    below 0x8A00 (a <= 0x7FFF);
//  * m = 0xFFFF for negative y, else 0;
//  * the entry's byte offset min(i2, 3326) + 3328 s (the negative half of the
//    table follows the positive one).
// gfx9 VOP3P encodings take no literal: the constants come in SGPRs, at most
// one per instruction.
struct GeluPair {
  uint32_t i2, m, off;
};
__device__ __forceinline__ GeluPair gelu_pair_index(uint32_t p) {
  GeluPair g;
  uint32_t t0;
  asm("v_pk_mad_u16 %[i2], %[p], 2, %[c0] op_sel_hi:[1,0,1]\n\t"
      "v_pk_ashrrev_i16 %[m], 15, %[p] op_sel_hi:[0,1]\n\t"
      "v_pk_min_u16 %[off], %[i2], %[c1]\n\t"
      "v_and_b32 %[t0], 0xd000d00, %[m]\n\t"
      "v_pk_add_u16 %[off], %[off], %[t0]"
      : [i2] "=&v"(g.i2), [m] "=&v"(g.m), [off] "=&v"(g.off), [t0] "=&v"(t0)
      : [p] "v"(p), [c0] "s"(0x8A008A00u), [c1] "s"(0x0CFE0CFEu));
  return g;
}

// GELU of a packed BF16 pair p given its two table entries t (packed the
// same way), per half:
//  * the entry where k < 0x8900, k = i2 for negative y and i2 + 0x7C01
//    (saturating) for positive y: the table's range, and for negative y also
//    every finite value past it (the clamped entry is -0);
//  * below the table (i2 >= 0x8A00) the BF16 rounding of y/2 (y * 0.5 in
//    fp32 is exact);
//  * otherwise (positive y past the table, -inf, NaN) y with bit 6 set for
//    negative y: +inf stays +inf, -inf gives 0xFFC0, NaNs stay quiet NaNs.
// The two tests are the sign bits of saturating differences (k - 0x900 and
// i2 - 0xA00), spread over the half by an arithmetic shift into bit masks
// for v_bfi_b32.
__device__ __forceinline__ uint32_t gelu_pair_select(uint32_t p, uint32_t t, const GeluPair& g) {
  uint32_t r, k, b2, lo, hi;
  asm("v_bfi_b32 %[k], %[m], 0, %[c0]\n\t"
      "v_pk_add_u16 %[k], %[i2], %[k] clamp\n\t"
      "v_pk_sub_u16 %[k], %[k], %[c1] clamp\n\t"
      "v_pk_ashrrev_i16 %[k], 15, %[k] op_sel_hi:[0,1]\n\t"
      "v_pk_sub_u16 %[b2], %[i2], %[c2] clamp\n\t"
      "v_pk_ashrrev_i16 %[b2], 15, %[b2] op_sel_hi:[0,1]\n\t"
      "v_lshlrev_b32 %[lo], 16, %[p]\n\t"
      "v_and_b32 %[hi], 0xffff0000, %[p]\n\t"
      "v_mul_f32 %[lo], 0.5, %[lo]\n\t"
      "v_mul_f32 %[hi], 0.5, %[hi]\n\t"
      "v_cvt_pk_bf16_f32 %[lo], %[lo], %[hi]\n\t"
      "v_and_or_b32 %[hi], %[m], %[c3], %[p]\n\t"
      "v_bfi_b32 %[lo], %[b2], %[lo], %[hi]\n\t"
      "v_bfi_b32 %[r], %[k], %[lo], %[t]"
      : [r] "=&v"(r), [k] "=&v"(k), [b2] "=&v"(b2), [lo] "=&v"(lo), [hi] "=&v"(hi)
      : [p] "v"(p), [t] "v"(t), [i2] "v"(g.i2), [m] "v"(g.m), [c0] "s"(0x7C017C01u),
        [c1] "s"(0x09000900u), [c2] "s"(0x0A000A00u), [c3] "s"(0x00400040u));
  return r;
}

// 128-byte LDS rows hold 8 chunks of 16 bytes; logical chunk c of row r sits
// at c ^ key(r). Weight rows are read in the permuted slot order (row slot
// 4 q + e of tile i is row 32 (i / 2) + 8 q + 4 (i % 2) + e), activation rows
// in order.
__device__ __forceinline__ int key_w(int r) { return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int key_a(int r) { return r & 7; }

// A workgroup's k-th item: its tile origin (in full-tile mode the last tile
// row and column end at M and N) and, for a GEMM split over K into `splits`
// parts, its part and that part's stages kb0 .. kb0 + kbn - 1 of the nk.
struct Item {
  int m0, n0, part, kb0, kbn;
};
template <bool kFull>
__device__ __forceinline__ Item item_of(const Sched& s, int k, int M, int N, int nk, int splits) {
  Item it;
  const int id = s.start + k * s.stride;
  const int T = s.tiles_m * s.tiles_n;
  it.part = splits == 1 ? 0 : id / T;
  tile_of<kBM, kBN, kGroupM>(s, id - it.part * T, it.m0, it.n0);
  if constexpr (kFull) {
    it.m0 = it.m0 < M - kBM ? it.m0 : M - kBM;
    it.n0 = it.n0 < N - kBN ? it.n0 : N - kBN;
  }
  it.kb0 = it.part * nk / splits;
  it.kbn = (it.part + 1) * nk / splits - it.kb0;
  return it;
}

__device__ __forceinline__ void mfma_all(v4i (&acc)[kTN][kTM], const v4i (&f)[kTN + kTM]) {
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f[i], f[kTN + j], acc[i][j], 0, 0, 0);
}

template <Epilogue kEpi, bool kFull>
__global__ __launch_bounds__(kThreads, 1)
void gemm_i8_pipelined(const int8_t* __restrict__ a, int64_t lda, const int8_t* __restrict__ w,
                       int64_t ldw, const float* __restrict__ a_scale,
                       const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
                       void* __restrict__ out, int64_t ldo, int M, int N, int K, int tiles_m,
                       int tiles_n, int splits) {
  constexpr bool kScales = kEpi != Epilogue::kInt32;
  constexpr bool kBias = epilogue_has_bias(kEpi);
  constexpr bool kGelu = epilogue_has_gelu(kEpi);
  // a tile's scales, then (with a bias) its biases
  constexpr int kBufBytes = kScaleBytes + (kBias ? kBiasBytes : 0);
  constexpr int kScaleLoads = kBias ? 2 : 1;   // wave-loads per wave per tile
  constexpr int kGeluBytes = kGelu ? kGeluTable * 2 : 0;
  __shared__ __attribute__((aligned(1024)))
  int8_t lds[kSlots * kSlotBytes + kScaleBufs * kBufBytes + kGeluBytes];
  int8_t* const scale_bufs = lds + kSlots * kSlotBytes;
  int8_t* const gelu_lds = scale_bufs + kScaleBufs * kBufBytes;

  // Items: the tiles, or with splits > 1 (INT32 partial sums only) one per
  // (K part, tile); part p's sums go to out + p * M * ldo.
  const Sched sc = make_sched(blockIdx.x, gridDim.x, tiles_m, tiles_n, tiles_m * tiles_n * splits);
  const int nk = K / kBK;                       // stages of the whole K
  if (sc.count == 0) return;
  if constexpr (kGelu) {
    // the GELU table; the prologue's barrier publishes it
    uint16_t* tab = reinterpret_cast<uint16_t*>(gelu_lds);
    for (int i = threadIdx.x; i < kGeluTable; i += kThreads) tab[i] = gelu_table_entry(i);
    wait_lgkmcnt0();
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;

  // ---- loader: only waves 0 .. kLoaderWaves-1 refill the ring (one per SIMD:
  // issuing the refills stalls the issuing wave, and the other wave of its
  // SIMD keeps the MFMAs fed meanwhile). Loader wave v's wave-load g fills
  // stage rows 8 (v + kLoaderWaves g) + [0, 8) of the weight half and then of
  // the activation half; lane -> row r_l + 8 kLoaderWaves g, physical chunk
  // lane % 8, logical chunk fixed per lane (the keys ignore row bits >= 5).
  constexpr int kRowStep = 8 * kLoaderWaves;
  const bool loader = wave < kLoaderWaves;
  const int r_l = 8 * (wave % kLoaderWaves) + (lane >> 3);
  const int p = lane & 7;
  const int cw = (p ^ key_w(r_l)) << 4, ca = (p ^ key_a(r_l)) << 4;
  // The tile's weight and activation row blocks as buffers. Full tiles: a
  // load's offset is the lane's row-0 offset plus 64 g rows and the stage's
  // K offset, both in an SGPR. Otherwise rows past N or M are clamped to the
  // last valid row (their sums duplicate it and are stored over it with
  // identical values).
  int ld_k = 0, ld_kt = 0, ld_nk = 0, ld_rvn = 0, ld_rvm = 0;
  const int vo_w = r_l * (int)ldw + cw, vo_a = r_l * (int)lda + ca;
  __amdgpu_buffer_rsrc_t ld_w, ld_a;
  auto load_tile = [&](int k) {
    const Item it = item_of<kFull>(sc, k, M, N, nk, splits);
    const int rn = (N - it.n0) < kBN ? (N - it.n0) : kBN;
    const int rm = (M - it.m0) < kBM ? (M - it.m0) : kBM;
    ld_rvn = rn - 1;
    ld_rvm = rm - 1;
    ld_nk = it.kbn;
    // the buffers start at the item's first K byte
    const int kb = it.kb0 * kBK;
    ld_w = buffer_rsrc(w + (int64_t)it.n0 * ldw + kb, (uint32_t)(rn * ldw - kb));
    ld_a = buffer_rsrc(a + (int64_t)it.m0 * lda + kb, (uint32_t)(rm * lda - kb));
  };
  load_tile(0);
  auto issue_next = [&](int slot) {
    if (!loader) return;
    int8_t* dst = lds + slot * kSlotBytes + (wave % kLoaderWaves) * 1024;
    const int koff = ld_kt * kBK;
#pragma unroll
    for (int g = 0; g < kLoads / 2; ++g) {
      const int r = r_l + kRowStep * g;
      if constexpr (kFull)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_w, (lds_void*)(dst + g * kRowStep * kBK), 16,
                                                 vo_w, koff + kRowStep * g * (int)ldw, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_w, (lds_void*)(dst + g * kRowStep * kBK), 16,
                                                 (r < ld_rvn ? r : ld_rvn) * (int)ldw + cw, koff,
                                                 0, 0);
    }
#pragma unroll
    for (int g = 0; g < kLoads / 2; ++g) {
      const int r = r_l + kRowStep * g;
      if constexpr (kFull)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_a,
                                                 (lds_void*)(dst + kBN * kBK + g * kRowStep * kBK),
                                                 16, vo_a, koff + kRowStep * g * (int)lda, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ld_a,
                                                 (lds_void*)(dst + kBN * kBK + g * kRowStep * kBK),
                                                 16, (r < ld_rvm ? r : ld_rvm) * (int)lda + ca,
                                                 koff, 0, 0);
    }
  };
  // Loader advance. It branches, so it runs at the top of a stage: placed after
  // the stage's code it would give the compiler a block past the branch into
  // which it sinks the next stage's fragment reads, away from the MFMAs they
  // should hide behind.
  auto advance_loader = [&]() {
    if (++ld_kt == ld_nk) {
      ld_kt = 0;
      if (++ld_k < sc.count) load_tile(ld_k);   // past the end: reloads of the last tile
    }
  };

  // Scales of tile k into buffer k % 3: waves 0-3 move 64 weight scales
  // each, waves 4-7 64 activation scales (one wave-load of one dword per
  // lane). Tile k + 1's scales go out when tile k starts; the buffer they
  // overwrite was last read by tile k - 2's epilogue, which every wave
  // finished before a barrier of tile k - 1.
  auto issue_scales = [&](int k) {
    const Item it = item_of<kFull>(sc, k, M, N, nk, splits);
    const int m0 = it.m0, n0 = it.n0;
    int8_t* buf = scale_bufs + (k % kScaleBufs) * kBufBytes;
    // a buffer over the whole scale vector; indices past the end are clamped
    // to its last element (clamped rows reuse row M-1's scale). The lane
    // offset is recomputed here rather than kept live across the tile.
    const int ln = lane_id();
    const int lim = wave < 4 ? N : M;
    int idx = (wave < 4 ? n0 + 64 * wave : m0 + 64 * (wave - 4)) + ln;
    idx = idx < lim ? idx : lim - 1;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(wave < 4 ? w_scale : a_scale, (uint32_t)(4 * lim));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + wave * 256), 4, 4 * idx, 0, 0,
                                             0);
    if constexpr (kBias) {
      // BF16 biases as dwords (pairs of channels): waves 0 and 1 bring the
      // tile's 128 dwords, the other waves the same again into space nothing
      // reads, so every wave issues the same loads
      const int nd = N >> 1;
      int di = (n0 >> 1) + 64 * (wave & 1) + ln;
      di = di < nd ? di : nd - 1;
      const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(bias, (uint32_t)(4 * nd));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(buf + kScaleBytes + wave * 256), 4,
                                               4 * di, 0, 0, 0);
    }
  };

  // ---- fragments: MFMA row slot ir = lane % 16 of W tile i maps to wave-local
  // channel 32 (i / 2) + 8 (ir / 4) + 4 (i % 2) + ir % 4, so lane (ir, kq)
  // holds channels 32 p + 8 kq .. 32 p + 8 kq + 7 of token ir + 16 j in tiles
  // 2 p and 2 p + 1 (p < 4): the four lanes of a token cover 32 consecutive
  // channels.
  const int ir = lane & 15, kq = lane >> 4;
  const int w_row0 = wn * 128 + 8 * (ir >> 2) + (ir & 3);
  const int a_row0 = kBN + wm * (16 * kTM) + ir;
  const int w_base = w_row0 * kBK, w_key = key_w(w_row0);
  const int a_base = a_row0 * kBK, a_key = key_a(a_row0 - kBN);
  auto read_frags = [&](v4i (&f)[kTN + kTM], int slot, int ks) {
    const int8_t* sb = lds + slot * kSlotBytes;
    const int cl = ks * 4 + kq;
    const int wo = w_base + ((cl ^ w_key) << 4), ao = a_base + ((cl ^ a_key) << 4);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
      f[i] = *reinterpret_cast<const v4i*>(sb + wo + (32 * (i >> 1) + 4 * (i & 1)) * kBK);
#pragma unroll
    for (int j = 0; j < kTM; ++j)
      f[kTN + j] = *reinterpret_cast<const v4i*>(sb + ao + j * 16 * kBK);
  };

  v4i acc[kTN][kTM];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  };
  zero_acc();
  v4i f0[kTN + kTM], f1[kTN + kTM];

  // ---- epilogue of tile k -----------------------------------------------------
  // ---- epilogue of tile k: lane constants recomputed (not held live) ------
  auto epilogue = [&](int k) {
    const int el = lane_id();
    const int ir = el & 15, kq = el >> 4;
    const Item it = item_of<kFull>(sc, k, M, N, nk, splits);
    const int m0 = it.m0, n0 = it.n0;
    const int n_wave = n0 + wn * 128;
    if (n_wave >= N) return;
    const int n_lane = n_wave + 8 * kq;
    const int m_lane = m0 + wm * (16 * kTM) + ir;
    if constexpr (kEpi == Epilogue::kInt32) {
      int32_t* o = reinterpret_cast<int32_t*>(out) + (int64_t)it.part * M * ldo;
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        int m = m_lane + 16 * j;
        if constexpr (!kFull) m = m < M ? m : M - 1;   // clamped rows hold row M-1's sums
        int32_t* dst = o + (int64_t)m * ldo + n_lane;
#pragma unroll
        for (int i = 0; i < kTN; ++i)
          *reinterpret_cast<v4i*>(dst + 32 * (i >> 1) + 4 * (i & 1)) = acc[i][j];
      }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      // byte offset of lane (ir, kq)'s first store within its row block:
      // token ir % 8, channels 32 (ir / 8) + 8 kq
      const uint32_t st_lane = (uint32_t)(((ir & 7) * (int)ldo + 32 * (ir >> 3) + 8 * kq) * 2);
      // the tile's scales, brought into LDS one tile ahead
      const uint32_t sbuf = lds_addr(scale_bufs + (k % kScaleBufs) * kBufBytes);
      float sa[kTM];
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        sa[j] = lds_read_f1(sbuf + 4 * (kBN + wm * (16 * kTM) + 16 * j + ir));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {          // stores p = 2 hf and 2 hf + 1
        // channels 32 p + 8 kq + e (e < 8) of the wave's 128
        const uint32_t swa = sbuf + 4 * (wn * 128 + 64 * hf + 8 * kq);
        v4f t0 = lds_read_f4(swa);
        v4f t1 = lds_read_f4(swa + 16);
        v4f t2 = lds_read_f4(swa + 128);
        v4f t3 = lds_read_f4(swa + 144);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3), "+v"(sa[0]), "+v"(sa[1]),
                       "+v"(sa[2]), "+v"(sa[3])
                     :
                     : "memory");
        const float sw[16] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3],
                              t2[0], t2[1], t2[2], t2[3], t3[0], t3[1], t3[2], t3[3]};
        uint32_t bw[kBias ? 8 : 1];
        if constexpr (kBias) {
          const uint32_t ba = sbuf + kScaleBytes + 2 * (wn * 128 + 64 * hf + 8 * kq);
          v4f b0 = lds_read_f4(ba), b1 = lds_read_f4(ba + 64);
          asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(b0), "+v"(b1) : : "memory");
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bw[e] = __float_as_uint(b0[e]);
            bw[4 + e] = __float_as_uint(b1[e]);
          }
        }
#pragma unroll
        for (int j = 0; j < kTM; ++j) {
          v4u pk[2];   // token m_lane + 16 j, channels 64 hf + 32 pp + 8 kq + [0, 8)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int p = 2 * hf + pp;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              v[e] = ((float)acc[2 * p + (e >> 2)][j][e & 3] * sa[j]) * sw[8 * pp + e];
            if constexpr (kBias) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                v[2 * q] = v[2 * q] + bf16_lo(bw[4 * pp + q]);
                v[2 * q + 1] = v[2 * q + 1] + bf16_hi(bw[4 * pp + q]);
              }
            }
            v4u packed;
            if constexpr (kGelu) {   // the FFN activation on the BF16 Linear output
              // the values rounded to BF16, packed in pairs as they are stored
              uint32_t y[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) y[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
              const uint32_t tab = lds_addr(gelu_lds);
              // the two entries of a pair, zero-extended (16-bit loads into
              // half a register do not keep the other half on this chip)
              uint32_t t[8];
              GeluPair g[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                g[q] = gelu_pair_index(y[q]);
                asm volatile("ds_read_u16 %0, %1" : "=v"(t[2 * q]) : "v"(tab + (g[q].off & 0xFFFFu)));
                asm volatile("ds_read_u16 %0, %1" : "=v"(t[2 * q + 1]) : "v"(tab + (g[q].off >> 16)));
              }
              asm volatile("s_waitcnt lgkmcnt(0)"
                           : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]),
                             "+v"(t[5]), "+v"(t[6]), "+v"(t[7])
                           :
                           : "memory");
#pragma unroll
              for (int q = 0; q < 4; ++q)
                packed[q] = gelu_pair_select(y[q], t[2 * q] | (t[2 * q + 1] << 16), g[q]);
            } else {
              packed = v4u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            }
            pk[pp] = packed;
          }
          // Whole 128-byte lines per store: lanes ir and ir ^ 8 of each
          // 16-lane row swap one value (DPP row rotate by 8), so store 0
          // writes tokens 16 j + 0..7 and store 1 tokens 16 j + 8..15, each
          // token's 64 channels (64 hf ..) by 8 lanes. Non-temporal stores of
          // half lines cost about a third more bytes past the L2.
          // Two bank-masked DPP moves per value: store 0 keeps pk[0] in lanes
          // 0-7 of each row and takes pk[1] of lanes 0-7 into lanes 8-15
          // (banks 2 and 3); store 1 keeps pk[1] in lanes 8-15 and takes
          // pk[0] of lanes 8-15 into lanes 0-7 (banks 0 and 1).
          v4u st0, st1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            st0[q] = (uint32_t)__builtin_amdgcn_update_dpp((int)pk[0][q], (int)pk[1][q], 0x128,
                                                           0xF, 0xC, false);
            st1[q] = (uint32_t)__builtin_amdgcn_update_dpp((int)pk[1][q], (int)pk[0][q], 0x128,
                                                           0xF, 0x3, false);
          }
          // Rows past M (clamped tiles only) hold exactly row M-1's sums
          // (their loads were clamped to it) and its scale, so they store row
          // M-1's values to row M-1: every lane issues its stores and the
          // per-tile store count stays fixed.
          // Non-temporal: the output streams past the caches instead of
          // evicting the activation and weight rows the next tiles read.
          if constexpr (kFull) {
            // a wave-uniform row-block address plus the lane's 32-bit offset
            // (the host keeps 256 output rows within 2^31 bytes), so the
            // stores take the scalar-base form with no 64-bit VALU address
            // arithmetic
            const char* blk = reinterpret_cast<const char*>(
                o + ((int64_t)(m0 + wm * (16 * kTM) + 16 * j) * ldo + n_wave + 64 * hf));
            char* b0 = const_cast<char*>(blk) + st_lane;
            char* b1 = const_cast<char*>(blk) + 16 * ldo + st_lane;
            __builtin_nontemporal_store(st0, reinterpret_cast<v4u*>(b0));
            __builtin_nontemporal_store(st1, reinterpret_cast<v4u*>(b1));
          } else {
            int m_st0 = m0 + wm * (16 * kTM) + 16 * j + (ir & 7), m_st1 = m_st0 + 8;
            m_st0 = m_st0 < M ? m_st0 : M - 1;
            m_st1 = m_st1 < M ? m_st1 : M - 1;
            const int col = n_wave + 64 * hf + 32 * (ir >> 3) + 8 * kq;
            __builtin_nontemporal_store(st0,
                                        reinterpret_cast<v4u*>(o + (int64_t)m_st0 * ldo + col));
            __builtin_nontemporal_store(st1,
                                        reinterpret_cast<v4u*>(o + (int64_t)m_st1 * ldo + col));
          }
        }
      }
    }
  };

  // The tile-start group (the previous tile's stores, then the next tile's
  // scale loads) goes out after the loads of the tile's second stage, so only
  // the tile's first barrier leaves it outstanding. Stores are counted only
  // when every wave stores a full tile (full-tile mode, or N a multiple of
  // 256); otherwise the wait covers them too, which is merely slower.
  const int stores_per_tile =
      (kEpi != Epilogue::kInt32 && (kFull || N % kBN == 0)) ? kStoresPerTile : 0;
  int pending_stores = 0;

  // ---- prologue: tile 0's scales; stages 0 and 1 in flight; fragments of
  // stage 0, K step 0 ----
  if constexpr (kScales) issue_scales(0);
  issue_next(0);
  advance_loader();
  issue_next(1);
  wait_vmcnt_le(loader ? kLoads : 0);    // stage 0 landed
  lds_barrier();
  read_frags(f0, 0, 0);

  // ---- main loop: per stage, K step 0 from f0 (read one step ahead) and K
  // step 1 from f1; the stage barrier sits between them. --------------------
  int s = 0;
  for (int k = 0; k < sc.count; ++k) {
    if (kScales && k + 1 < sc.count) {
      issue_scales(k + 1);
      pending_stores += kScaleLoads;
    }
    const int kbn = item_of<kFull>(sc, k, M, N, nk, splits).kbn;
    for (int kt = 0; kt < kbn; ++kt, ++s) {
      const int slot = s & 1;
      advance_loader();                    // to stage s+2
      // K step 0 (f0), K step 1's fragments read between its MFMAs
      read_frags(f1, slot, 1);
      mfma_all(acc, f0);
#pragma unroll
      for (int q = 0; q < kTN + kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kTN * kTM - (kTN + kTM), 0);
      __builtin_amdgcn_sched_barrier(0);
      // Every stage has its barrier and refills a slot, past the last stage
      // with reloads of a valid stage into slots nothing reads again, so the
      // code between barriers has no branches and the refill loads and the
      // next stage's fragment reads interleave with K step 1's MFMAs.
      wait_lgkmcnt0();                     // this wave is done reading slot `slot`
      wait_vmcnt_le(pending_stores);       // stage s+1 has landed
      lds_barrier();                       // ... for every wave; slot `slot` is free
      __builtin_amdgcn_sched_barrier(0);
      pending_stores = 0;
      issue_next(slot);                    // stage s+2 reuses this slot
      read_frags(f0, slot ^ 1, 0);
      mfma_all(acc, f1);
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < kTN + kTM; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kTN * kTM - kLoads - (kTN + kTM), 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    epilogue(k);
    if constexpr (kEpi == Epilogue::kInt32) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    pending_stores = stores_per_tile;
    zero_acc();
  }
  // LDS DMA still in flight must land before the workgroup's LDS is released.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace pipe

// Compute units of the current device, queried once per device. Calls from
// several host threads may race to fill an entry; they store the same value,
// and the entries are atomics so that this is well defined.
int device_cu_count() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_gemm_pipelined(Epilogue epi, const int8_t* a, int64_t lda, const int8_t* w,
                                 int64_t ldw, const float* a_scale, const float* w_scale,
                                 const uint16_t* bias, void* out, int64_t ldo, int64_t M,
                                 int64_t N, int64_t K, hipStream_t st, int splits) {
  if (splits < 1 || (splits > 1 && epi != Epilogue::kInt32) || splits > (int)(K / pipe::kBK))
    return hipErrorInvalidValue;
  const int tiles_m = (int)((M + pipe::kBM - 1) / pipe::kBM);
  const int tiles_n = (int)((N + pipe::kBN - 1) / pipe::kBN);
  const int64_t tiles = (int64_t)tiles_m * tiles_n * splits;
  const int cus = device_cu_count();
  const int grid = (int)(tiles < cus ? tiles : cus);
  const dim3 block(pipe::kThreads);
  // full-tile mode needs at least one whole tile in each direction
  const bool full = M >= pipe::kBM && N >= pipe::kBN;
#define W8A8_PIPE_LAUNCH(E, F)                                                           \
  hipLaunchKernelGGL((pipe::gemm_i8_pipelined<E, F>), dim3(grid), block, 0, st, a, lda, w, \
                     ldw, a_scale, w_scale, bias, out, ldo, (int)M, (int)N, (int)K, tiles_m,  \
                     tiles_n, splits)
#define W8A8_PIPE_LAUNCH2(E)           \
  if (full) W8A8_PIPE_LAUNCH(E, true); \
  else W8A8_PIPE_LAUNCH(E, false)
  switch (epi) {
    case Epilogue::kInt32: W8A8_PIPE_LAUNCH2(Epilogue::kInt32); break;
    case Epilogue::kPostscaleBf16: W8A8_PIPE_LAUNCH2(Epilogue::kPostscaleBf16); break;
    case Epilogue::kPostscaleBiasBf16: W8A8_PIPE_LAUNCH2(Epilogue::kPostscaleBiasBf16); break;
    case Epilogue::kPostscaleGeluBf16: W8A8_PIPE_LAUNCH2(Epilogue::kPostscaleGeluBf16); break;
    case Epilogue::kPostscaleBiasGeluBf16:
      W8A8_PIPE_LAUNCH2(Epilogue::kPostscaleBiasGeluBf16);
      break;
    default: return hipErrorInvalidValue;
  }
#undef W8A8_PIPE_LAUNCH2
#undef W8A8_PIPE_LAUNCH
  return hipGetLastError();
}

}  // namespace w8a8
