// Engine-clock probe for measurements: the matrix-core peak scales with the
// engine clock, so a throughput is judged against the clock the chip held
// while the work ran.  Each one-wave workgroup counts the shader clock
// (s_memtime) against the constant 100 MHz real-time counter (s_memrealtime)
// for a given span of real time; run beside other work on a second stream it
// measures the clock under that load.  Workgroup w lands on XCD w % 8.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* __restrict__ out, unsigned long long span,
                                                         int max_iters) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long r1 = r0;
    for (int i = 0; i < max_iters && r1 - r0 < span; ++i) {   // bounded: ends after max_iters sleeps at most
        __builtin_amdgcn_s_sleep(8);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

hipError_t launch_clock_probe(unsigned long long* out, int n_wg, double seconds, hipStream_t st) {
    const unsigned long long span = (unsigned long long)(seconds * 1e8);   // real-time ticks (100 MHz)
    // s_sleep 8 waits about 8 x 64 cycles: at 3 GHz or less one iteration is
    // at least 0.17 us, so 64 iterations per microsecond bound the loop
    const double iters = seconds * 1e6 * 64.0 + 1024.0;
    const int max_iters = iters > 2e9 ? 2000000000 : (int)iters;
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)n_wg), dim3(64), 0, st, out, span, max_iters);
    return hipGetLastError();
}

}  // namespace fa
