// Shader-clock sampling for measurements (not part of the attention method).
//
// Each workgroup of one wave records, from its first lane, the 100 MHz real-time
// counter (s_memrealtime), the shader-cycle counter (s_memtime, which advances
// at the current shader clock), and the XCC and HW_ID hardware registers that
// say where it ran.  Launched just before and just after a timed region on the
// same stream, two samples from one XCD give that XCD's average shader clock
// over the region: (cycles_after - cycles_before) / (realtime_after -
// realtime_before) x 100 MHz.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu_kernels.h"

namespace hstu {
namespace {

__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t* out) {
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    const uint64_t cy = __builtin_amdgcn_s_memtime();
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
    const uint32_t hwid = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_REG_HW_ID
    if (threadIdx.x == 0) {
        uint64_t* o = out + 4 * (size_t)blockIdx.x;
        o[0] = rt;
        o[1] = cy;
        o[2] = xcc;
        o[3] = hwid;
    }
}

}  // namespace

hipError_t launch_clock_sample(uint64_t* out, int count, hipStream_t stream) {
    hipLaunchKernelGGL(clock_sample_kernel, dim3((unsigned)count), dim3(64), 0, stream, out);
    return hipGetLastError();
}

}  // namespace hstu
