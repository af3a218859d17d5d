// bench_clock.hip - shader-clock probe for bench.py (measurement only; not
// part of libfa).
//
// One wave reads the shader-clock counter (s_memtime, which advances at the
// clock the compute units actually run at) and the constant-rate counter
// (s_memrealtime, hipDeviceAttributeWallClockRate: 100 MHz on MI355X) at the
// start and the end of a window of `ticks` constant-rate ticks, sleeping in
// between. Launched on a side stream while a kernel runs back to back on
// the main stream, it gives the clock that kernel holds, so a fraction of
// the datasheet peak (quoted at 2.4 GHz) can also be stated at the measured
// clock: the roofline of [Capstone §1.2] scales with it.
#include <hip/hip_runtime.h>

namespace {

__global__ void clock_probe_kernel(unsigned long long* out,
                                   unsigned long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r = r0;
  // bounded: at most 2^24 sleeps of ~640 cycles each, whatever `ticks` is
  for (int it = 0; it < (1 << 24); ++it) {
    __builtin_amdgcn_s_sleep(10);
    r = __builtin_amdgcn_s_memrealtime();
    if (r - r0 >= ticks) break;
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
}

}  // namespace

extern "C" {

// Enqueue the probe on `stream`: out (device, 2 x uint64) receives the
// shader-clock cycles and the constant-rate ticks of the window.
int bench_clock_probe(unsigned long long* out, unsigned long long ticks,
                      void* stream) {
  if (out == nullptr) return -1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out, ticks);
  return (int)hipGetLastError();
}

// Rate of the constant-rate counter in kHz (0 if it cannot be read).
int bench_clock_wall_rate_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) !=
      hipSuccess)
    return 0;
  return khz;
}

}  // extern "C"
