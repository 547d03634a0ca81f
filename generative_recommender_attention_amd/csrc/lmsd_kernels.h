// Launch-side view of the LMSD kernels: their parameter block and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

struct LmsdParams {
    int64_t n;                 // rows
    int32_t d;                 // values per row, 8 <= d < 1024, d % 8 == 0
    int32_t segs;              // output segments S = 1 + concat_u + concat_x
    float eps;
    float inv_d;               // 1 / d
    int32_t silu_u, concat_u, concat_x;
    const uint16_t* x;         // (n, d) bf16, row stride x_stride
    const uint16_t* u;         // (n, d) bf16, row stride u_stride
    const uint16_t* weight;    // (d) bf16
    const uint16_t* bias;      // (d) bf16
    int64_t x_stride, u_stride;
    // forward
    uint16_t* y;               // (n, S d) bf16, contiguous
    float* mean;               // (n): written by the forward, read by the backward
    float* rstd;               // (n): likewise
    // backward
    const uint16_t* dy;        // (n, S d) bf16, row stride dy_stride
    int64_t dy_stride;
    uint16_t* dx;              // (n, d) bf16, row stride dx_stride
    uint16_t* du;              // (n, d) bf16, row stride du_stride
    int64_t dx_stride, du_stride;
    uint16_t* dweight;         // (d) bf16, or null when not computed
    uint16_t* dbias;           // (d) bf16
    float* work;               // parts rows of part_stride fp32: [dbias partial | dweight partial]
    int64_t part_stride;
};

// Largest number of workgroup partials of the backward's column sums.
constexpr int kLmsdMaxParts = 1024;

// Workgroups (= partial rows) the backward launches for n rows of d values.
int lmsd_bwd_parts(int64_t n, int d);

// Largest d (d < 1024, d % 8 == 0) and the bytes of column partials the backward
// can need: kLmsdMaxParts rows of [dbias | dweight], 2 d fp32 each (8,323,072 bytes).
constexpr int kLmsdMaxD = 1016;
constexpr size_t kLmsdScratchBytes = (size_t)kLmsdMaxParts * 2 * kLmsdMaxD * sizeof(float);

// Device address, on the current device, of the library's own kLmsdScratchBytes of
// scratch for the backward's column partials (looked up once per device).
hipError_t lmsd_scratch(void** ptr);

hipError_t launch_lmsd_fwd(const LmsdParams& p, hipStream_t stream);
hipError_t launch_lmsd_bwd(const LmsdParams& p, int parts, hipStream_t stream);

}  // namespace hstu
