// Building blocks shared by the persistent, software-pipelined INT8 GEMM
// kernels for gfx950: the XCD-aware tile schedule, buffer descriptors for
// loads that write LDS directly, and the waits and LDS reads the pipelines
// need written so that the compiler adds no waits of its own.
#pragma once

#include "device_common.hpp"

namespace w8a8 {
namespace pipe {

constexpr int kXcds = 8;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmemRead = 0x020,
              kSchedDsRead = 0x100;

typedef __attribute__((address_space(3))) void lds_void;
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n) for a run-time n, rounded down (waiting longer is safe).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  if (n >= 17) asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
  else if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n >= 15) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
  else if (n >= 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
  else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  else if (n >= 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_waitcnt vmcnt(N) for a compile-time N.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A workgroup's work items: logical ids start + k * stride, k < count. Workgroup
// b runs on XCD b % 8; each XCD owns a contiguous range of logical ids, so
// the rows its tiles share stay in that XCD's L2. Items default to the tiles;
// a split-K GEMM has one item per (K part, tile), the part changing slowest.
struct Sched {
  int start, stride, count, tiles_m, tiles_n;
};

__device__ __forceinline__ Sched make_sched(int b, int grid, int tiles_m, int tiles_n,
                                            int items = -1) {
  Sched s;
  s.tiles_m = tiles_m;
  s.tiles_n = tiles_n;
  const int T = items < 0 ? tiles_m * tiles_n : items;
  const int x = b % kXcds, j = b / kXcds;
  const int nwg = grid / kXcds + (x < grid % kXcds ? 1 : 0);     // workgroups on XCD x
  const int tx = T / kXcds + (x < T % kXcds ? 1 : 0);            // tiles of XCD x
  const int sx = x * (T / kXcds) + (x < T % kXcds ? x : T % kXcds);
  s.start = sx + j;
  s.stride = nwg;
  s.count = j < tx ? (tx - j + nwg - 1) / nwg : 0;
  return s;
}

// M-grouped order: groups of kGroupM tile rows, n fastest within a group.
// tile_of maps a tile id t < tiles_m * tiles_n; tile_mn a workgroup's k-th
// item when the items are the tiles.
template <int kBM, int kBN, int kGroupM>
__device__ __forceinline__ void tile_of(const Sched& s, int t, int& m0, int& n0) {
  const int span = kGroupM * s.tiles_n;
  const int g = t / span;
  const int first = g * kGroupM;
  const int gs = (s.tiles_m - first) < kGroupM ? (s.tiles_m - first) : kGroupM;
  const int in = t - g * span;
  m0 = (first + in % gs) * kBM;
  n0 = (in / gs) * kBN;
}

template <int kBM, int kBN, int kGroupM>
__device__ __forceinline__ void tile_mn(const Sched& s, int k, int& m0, int& n0) {
  tile_of<kBM, kBN, kGroupM>(s, s.start + k * s.stride, m0, n0);
}

// Raw buffer resource over [base, base + bytes): the address of a load is an
// SGPR base plus a 32-bit lane offset plus an SGPR offset, so issuing it costs
// no 64-bit VALU arithmetic (and anything past the end would read as zero).
// Word 3 is the gfx9-family raw-buffer descriptor encoding.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

// Lane index, recomputed where needed: the empty asm keeps the compiler from
// merging it with earlier copies, so values derived from it for the tile-level
// code are not held live across the stage loop.
__device__ __forceinline__ int lane_id() {
  int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

// LDS reads of scales. Written as instructions the compiler does not
// analyse: otherwise it cannot tell them apart from the LDS targets of the
// loads still in flight and waits for all of those first, draining the
// pipeline. The data they read is published by the stage barriers, and the
// caller waits for the reads with an lgkmcnt wait that names the results.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ v4f lds_read_f4(uint32_t addr) {
  v4f v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ float lds_read_f1(uint32_t addr) {
  float v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

}  // namespace pipe
}  // namespace w8a8
