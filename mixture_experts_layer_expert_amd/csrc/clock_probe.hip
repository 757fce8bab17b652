// Shader-clock probe: measures the core clock the GPU holds while other
// work runs, for reporting a kernel's throughput against the peak at the
// clock actually sustained.
//
// Each one-wave workgroup waits `delay` ticks of the 100 MHz real-time
// counter, then reads the shader clock counter (s_memtime) and the real-time
// counter (s_memrealtime) at both ends of a `window`-tick interval.  The
// clock is (shader cycles) / (real-time ticks) * 100 MHz.  Both waits are
// bounded by the real-time counter, which always advances, and the host
// caps delay + window.  The wave sleeps between reads, so it takes almost
// no issue slots from work sharing its compute unit.
#include "moe_internal.h"

namespace moe {
namespace {

// Both counters are read with the wait for the scalar load inside the same
// asm block, so the result register is complete when the block ends and
// the compiler cannot move the read.
__device__ inline uint64_t realtime_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
  return t;
}
__device__ inline uint64_t shader_clock_now() {
  uint64_t t;
  asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
  return t;
}

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t delay, uint64_t window, uint64_t* stamps) {
  const uint64_t r0 = realtime_now();
  uint64_t r = r0;
  while (r - r0 < delay) {
    __builtin_amdgcn_s_sleep(8);
    r = realtime_now();
  }
  const uint64_t c1 = shader_clock_now();
  const uint64_t r1 = realtime_now();
  r = r1;
  while (r - r1 < window) {
    __builtin_amdgcn_s_sleep(8);
    r = realtime_now();
  }
  const uint64_t c2 = shader_clock_now();
  const uint64_t r2 = realtime_now();
  if (threadIdx.x == 0) {
    uint64_t* o = stamps + 4 * (size_t)blockIdx.x;
    o[0] = r1;
    o[1] = r2;
    o[2] = c1;
    o[3] = c2;
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_clock_probe(int32_t blocks, double delay_us, double window_us, uint64_t* stamps,
                               moe_stream_t stream) {
  if (blocks < 1 || blocks > 65536 || !stamps) return MOE_ERR_INVALID_ARG;
  if (!(delay_us >= 0.0) || !(window_us > 0.0) || delay_us + window_us > 100000.0) return MOE_ERR_INVALID_ARG;
  // the real-time counter runs at 100 MHz: 100 ticks per microsecond
  const uint64_t delay = (uint64_t)(delay_us * 100.0), window = (uint64_t)(window_us * 100.0) + 1;
  hipLaunchKernelGGL(moe::clock_probe_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream, delay, window,
                     stamps);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
