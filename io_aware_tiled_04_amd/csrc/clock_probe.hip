// Shader-clock probe for the bench (not part of the attention ABI).
//
// One wave spins for `ticks` ticks of the constant-rate real-time counter
// (s_memrealtime) and counts the shader-clock cycles (s_memtime) that pass
// meanwhile; the bench launches it on a second stream while the attention
// kernel runs, so the ratio is the clock the chip holds under that load (on
// the XCD the probe lands on).  The loop always ends: the real-time counter
// only moves forward.  s_sleep keeps the spinning wave from taking issue
// slots from the kernel beside it.
#include <hip/hip_runtime.h>

#include <stdint.h>

extern "C" __global__ __launch_bounds__(64) void shader_clock_probe(unsigned long long* out, unsigned long long ticks) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    unsigned long long t1 = t0;
    while (t1 - t0 < ticks) {
        __builtin_amdgcn_s_sleep(8);
        t1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[0] = c1 - c0;
        out[1] = t1 - t0;
    }
}

// Launch the probe on `stream`: out (device, 2 x uint64) receives the
// shader-clock cycles and the real-time ticks of the window.
extern "C" int fa_bench_clock_probe(void* out, unsigned long long ticks, hipStream_t stream) {
    if (!out) return -1;
    void* args[] = {&out, &ticks};
    return hipLaunchKernel((const void*)shader_clock_probe, dim3(1), dim3(64), args, 0, stream) == hipSuccess ? 0 : -6;
}
