// fa_clock_probe.hip -- measurement helper for the benchmark (libfa_clock.so),
// not part of the attention library.
//
// The shader clock the GPU actually runs at while a workload executes: one
// wavefront, launched on a side stream while the workload's kernels are in
// flight, spins for a window of the 100 MHz real-time counter and counts
// shader clock cycles (s_memtime) over the same window.  Under a board power
// limit the clock sits below the frequency the published peak assumes, so
// the benchmark reports both.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void clock_probe_kernel(unsigned long long *out, unsigned long long window)
{
    if (threadIdx.x != 0) return;
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    while (r1 - r0 < window) r1 = __builtin_amdgcn_s_memrealtime();  // ends: the counter always advances
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    out[0] = t1 - t0;
    out[1] = r1 - r0;
}

}  // namespace

// out: device buffer of 2 uint64 (shader cycles, 100 MHz ticks) written by
// the probe; window_ticks: window length in 100 MHz ticks (>= 1); stream:
// hipStream_t to launch on.  Returns 0, or 1 if the launch was rejected.
extern "C" __attribute__((visibility("default"))) int fa_clock_probe(void *out,
                                                                      unsigned long long window_ticks,
                                                                      void *stream)
{
    if (!out || window_ticks == 0) return 1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       (unsigned long long *)out, window_ticks);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
