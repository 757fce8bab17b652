// Shader-clock probe: measures the core clock the GPU holds while other
// work runs, for reporting a kernel's throughput against the peak at the
// clock actually sustained.
//
// Each one-wave workgroup waits `delay` ticks of the 100 MHz real-time
// counter (s_memrealtime), then runs `iters` blocks of 1024 dependent
// v_add_u32 and reads the real-time counter again.  A wave64 VALU
// instruction occupies the 16-lane SIMD for 4 clocks, and each add needs the
// previous one's result, so the chain advances one add per 4 shader clocks:
// clock = 4096 * iters / (elapsed ticks / 100 MHz).  The loop's own
// branch and counter add about 28 clocks per 4096, which reads the clock
// 0.7% low.  (The s_memtime counter
// is not used: its rate relative to the shader clock varies.)  The wait is
// bounded by the real-time counter, which always advances, and the chain by
// its fixed length; the host bounds both.
#include "moe_internal.h"

namespace moe {
namespace {

// The read of the counter waits for its own result inside the same asm
// block, so the compiler can neither move it nor reuse the register early.
__device__ inline uint64_t realtime_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
  return t;
}

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t delay, int iters, uint64_t* stamps) {
  const uint64_t r0 = realtime_now();
  uint64_t r = r0;
  while (r - r0 < delay) {
    __builtin_amdgcn_s_sleep(8);
    r = realtime_now();
  }
  uint32_t x = threadIdx.x;
  const uint64_t r1 = realtime_now();
  for (int i = 0; i < iters; ++i) asm volatile(".rept 1024\n\tv_add_u32 %0, 1, %0\n\t.endr" : "+v"(x));
  const uint64_t r2 = realtime_now();
  if (threadIdx.x == 0) {
    uint64_t* o = stamps + 4 * (size_t)blockIdx.x;
    o[0] = r1;
    o[1] = r2;
    o[2] = (uint64_t)iters * 1024u;  // adds in the chain
    o[3] = x;                      // keeps the chain live
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_clock_probe(int32_t blocks, double delay_us, int32_t iters, uint64_t* stamps,
                               moe_stream_t stream) {
  if (blocks < 1 || blocks > 65536 || !stamps) return MOE_ERR_INVALID_ARG;
  if (!(delay_us >= 0.0) || delay_us > 100000.0 || iters < 1 || iters > (1 << 16)) return MOE_ERR_INVALID_ARG;
  // the real-time counter runs at 100 MHz: 100 ticks per microsecond
  const uint64_t delay = (uint64_t)(delay_us * 100.0);
  hipLaunchKernelGGL(moe::clock_probe_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream, delay, (int)iters,
                     stamps);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
