// Main-loop ceiling probe for the post-scale INT8 GEMM (a measurement aid,
// not part of the C ABI in include/).
//
// It runs the inner loop of the 256 x 256 block-tile GEMM on its own: a
// 2-slot LDS ring of 128-byte K stages filled by buffer loads that write LDS
// directly, fragments read one 64-byte K step ahead, and 8 waves of 8 x 4
// v_mfma_i32_16x16x64_i8 accumulators (128 x 64 outputs per wave), one stage
// barrier per stage. There is no epilogue and no tile change, and the
// operands come from a 2 MiB buffer that stays in L2, so the rate it reaches
// bounds what the full kernel can reach with the same loop. Run once on
// constant and once on random operands, it shows how much of the gap to the
// rated MFMA peak is set by the power the operand data draws rather than by
// the instruction schedule.
//
// Buffer layout: rows of 4096 bytes; rows 0..255 stand for a weight tile,
// rows 256..511 for an activation tile; stage s reads bytes
// (128 s) mod 4096 .. +127 of every row.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = 4096, kRows = 512;
constexpr int64_t kSrcBytes = (int64_t)kRowBytes * kRows;   // 2 MiB
constexpr int kSlotBytes = 65536;                            // 512 rows x 128 bytes
constexpr int kThreads = 512;
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// kRefill = false leaves the ring as the prologue filled it (the fragment
// reads and MFMAs then run on stale data): the loop without its refills.
template <bool kRefill>
__global__ __launch_bounds__(kThreads, 1) void mainloop(const int8_t* __restrict__ src, int stages,
                                                        int32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[2 * kSlotBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave >> 2, wm = wave & 3;
  // refill: each wave-load moves 8 rows x 128 bytes; lane (row r_l, 16-byte
  // chunk p) lands in LDS at chunk p ^ (r_l & 7) of its row
  const int r_l = 8 * wave + (lane >> 3), p = lane & 7;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (uint32_t)kSrcBytes);
  const int vo = r_l * kRowBytes + ((p ^ (r_l & 7)) << 4);
  auto issue = [&](int s) {
    const int koff = (s * 128) & (kRowBytes - 1);
    int8_t* dst = lds + (s & 1) * kSlotBytes + wave * 1024;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + g * 8192), 16, vo,
                                               koff + 64 * g * kRowBytes, 0, 0);
  };
  // fragments: lane (ir, kq) holds 16 K bytes (chunk 4 ks + kq) of row ir + 16 t
  const int ir = lane & 15, kq = lane >> 4;
  const int wrow = wn * 128 + ir, arow = 256 + wm * 64 + ir;
  v4i fw[2][8], fa[2][4];
  auto read_frags = [&](int s, int ks) {
    const int8_t* sb = lds + (s & 1) * kSlotBytes;
    const int c = ((ks * 4 + kq) ^ (ir & 7)) << 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) fw[ks][i] = *reinterpret_cast<const v4i*>(sb + (wrow + 16 * i) * 128 + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) fa[ks][j] = *reinterpret_cast<const v4i*>(sb + (arow + 16 * j) * 128 + c);
  };
  v4i acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  auto mfma = [&](int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[ks][i], fa[ks][j], acc[i][j], 0, 0, 0);
  };

  issue(0);
  issue(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  read_frags(0, 0);
  for (int s = 0; s < stages; ++s) {
    // K step 0; K step 1's fragments are read between its MFMAs
    read_frags(s, 1);
    mfma(0);
#pragma unroll
    for (int q = 0; q < 12; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 20, 0);
    __builtin_amdgcn_sched_barrier(0);
    // stage s+1 has landed and every wave is done with slot s
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kRefill) issue(s + 2);
    // K step 1; the next stage's first fragments are read between its MFMAs
    read_frags(s + 1, 0);
    mfma(1);
    if (kRefill) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 12; ++q) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kRefill ? 12 : 20, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // DMA still in flight must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int x = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) x ^= acc[i][j][0] ^ acc[i][j][1] ^ acc[i][j][2] ^ acc[i][j][3];
  sink[blockIdx.x * kThreads + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// Workgroups one launch runs: one per compute unit of the current device
// (0 if it cannot be read). The sink must hold workgroups * 512 int32.
int w8a8_probe_mainloop_workgroups() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n > 0 ? n : 0;
}

// src: device buffer of at least 2 MiB (see the layout above); stages >= 1;
// refill 0 or 1; sink: device buffer of at least workgroups * 512 int32
// (one value per thread, so the work is not dead code). Returns 0 on
// success, 1 for bad arguments (nothing is launched), 2 if the launch fails.
int w8a8_probe_mainloop(const int8_t* src, int64_t src_bytes, int stages, int refill,
                        int32_t* sink, int64_t sink_elems, hipStream_t stream) {
  const int grid = w8a8_probe_mainloop_workgroups();
  if (!src || !sink || src_bytes < kSrcBytes || stages < 1 || (refill != 0 && refill != 1) ||
      grid < 1 || sink_elems < (int64_t)grid * kThreads)
    return 1;
  if (refill)
    mainloop<true><<<grid, kThreads, 0, stream>>>(src, stages, sink);
  else
    mainloop<false><<<grid, kThreads, 0, stream>>>(src, stages, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
