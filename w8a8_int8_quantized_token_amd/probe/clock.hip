// Shader-clock stamps (a measurement aid, not part of the C ABI in include/).
//
// One workgroup per compute unit records, from its first lane: the hardware
// id of the CU it runs on (XCC, shader engine, shader array, CU), the shader
// clock counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime). Launched once before and once after a timed region on the
// same stream, the records of the same CU give the average shader clock over
// that region: (memtime_after - memtime_before) / (realtime_after -
// realtime_before) * 100 MHz.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

// s_getreg operands: hardware register id, offset 0, 32 bits.
constexpr int kHwRegHwId = 4;      // HW_ID: CU_ID [11:8], SH_ID [12], SE_ID [15:13] on gfx9
constexpr int kHwRegXccId = 20;    // XCC_ID [3:0] on gfx94x / gfx950
constexpr int kGetreg32 = (31 << 11);

__global__ __launch_bounds__(64) void clock_stamp(int64_t* __restrict__ out) {
  const uint32_t hw = __builtin_amdgcn_s_getreg(kGetreg32 | kHwRegHwId);
  const uint32_t xcc = __builtin_amdgcn_s_getreg(kGetreg32 | kHwRegXccId);
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    int64_t* o = out + 4 * (int64_t)blockIdx.x;
    o[0] = (int64_t)((xcc & 0xFu) << 8 | ((hw >> 8) & 0xFFu));   // XCC, SE, SH, CU
    o[1] = (int64_t)t;
    o[2] = (int64_t)r;
    o[3] = (int64_t)hw;
  }
}

}  // namespace

extern "C" {

// Writes 4 int64 per workgroup (CU key, memtime, memrealtime, raw HW_ID) for
// `workgroups` workgroups into out (at least 4 * workgroups elements).
// Returns 0 on success, 1 for bad arguments (nothing launched), 2 if the
// launch fails.
int w8a8_probe_clock_stamp(int64_t* out, int64_t out_elems, int workgroups, hipStream_t stream) {
  if (!out || workgroups < 1 || out_elems < 4 * (int64_t)workgroups) return 1;
  clock_stamp<<<workgroups, 64, 0, stream>>>(out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
