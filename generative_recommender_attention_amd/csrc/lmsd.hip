// HSTU LayerNorm-multiply-SiLU (LMSD) forward and backward on gfx950.
//
// Per row of N rows of D values (HSTU LMSD page, "Overview" equations; dropout
// off):
//     mean, rstd = 1 / sqrt(var + eps) (biased variance),  xh = (x - mean) rstd
//     l = xh weight + bias,  a = SiLU(u) or u,
//     y = [a if concat_u, x if concat_x, l a]
// and the page's explicit backward from dy, x, u, weight, bias and the saved
// mean and rstd (chain rule on the same equations):
//     dl = g a,  da = g l (+ ga),  du = da SiLU'(u) or da,
//     dxh = dl weight,  dx = rstd (dxh - mean(dxh) - xh mean(dxh xh)) (+ gx),
//     dweight = sum_rows dl xh,  dbias = sum_rows dl.
//
// The op moves each element once and does a few flops on it, so it is bound by
// HBM bandwidth; the kernels aim at streaming every byte once with enough
// loads in flight.  Layout: a row is D / 8 16-byte vectors; a group of LPR
// lanes (LPR = the power of two at or above D / 8, at most 64) owns one row,
// each lane VPL vectors (VPL = 2 only for D > 512), so a wave holds 64 / LPR
// rows and every global access is a 16-byte load or store per lane.  Row sums
// are butterfly reductions inside the lane group.  All arithmetic is fp32; the
// outputs are rounded to bf16 (nearest-even), the statistics stay fp32.
//
// Forward: one row group per wave, grid over the rows.  Backward: a persistent
// grid of G workgroups (G fixed by N and D on the host) walks the row groups;
// each lane accumulates its columns' dweight / dbias terms over its rows in
// registers, the workgroup sums its waves through LDS and writes one partial
// row per workgroup to the caller's workspace; a second kernel adds the G
// partials column by column, spread over 16 waves per column block, in a fixed
// order (deterministic).
#include <mutex>

#include "hstu_device.h"
#include "lmsd_kernels.h"

namespace hstu {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sigmoid(float s) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-s * kLog2e)); }

__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

// Sum over the LPR lanes of a row group (aligned groups of consecutive lanes).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int LPR, int VPL>
__global__ __launch_bounds__(256) void lmsd_fwd_kernel(LmsdParams p) {
    constexpr int RPW = 64 / LPR;  // rows per wave
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t row = wave * RPW + lane / LPR;
    const bool live = row < p.n;
    const int64_t r = live ? row : p.n - 1;  // dead lanes recompute the last row and store nothing
    HSTU_DCHECK(r >= 0 && r < p.n, kDbgLmsd);
    const int nvec = p.d / 8;

    float x[VPL][8], u[VPL][8];
    bool has[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = sub + k * LPR;
        has[k] = v < nvec;
        const int vv = has[k] ? v : 0;
        unpack8(ld_global16(p.x + r * p.x_stride + 8 * vv), x[k]);
        unpack8(ld_global16(p.u + r * p.u_stride + 8 * vv), u[k]);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        if (has[k])
#pragma unroll
            for (int i = 0; i < 8; ++i) s += x[k][i];
    const float mean = group_sum<LPR>(s) * p.inv_d;
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
        if (has[k])
#pragma unroll
            for (int i = 0; i < 8; ++i) q += (x[k][i] - mean) * (x[k][i] - mean);
    const float var = group_sum<LPR>(q) * p.inv_d;
    const float rstd = 1.0f / __builtin_sqrtf(var + p.eps);

    uint16_t* yr = p.y + r * (int64_t)p.segs * p.d;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        if (!live || !has[k]) continue;
        const int v = sub + k * LPR;
        float w[8], b[8], a[8], o[8];
        unpack8(ld_global16(p.weight + 8 * v), w);
        unpack8(ld_global16(p.bias + 8 * v), b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = p.silu_u ? u[k][i] * sigmoid(u[k][i]) : u[k][i];
            o[i] = ((x[k][i] - mean) * rstd * w[i] + b[i]) * a[i];
        }
        int seg = 0;
        if (p.concat_u) *reinterpret_cast<uint4*>(yr + (seg++) * p.d + 8 * v) = pack8(a);
        if (p.concat_x) *reinterpret_cast<uint4*>(yr + (seg++) * p.d + 8 * v) = pack8(x[k]);
        *reinterpret_cast<uint4*>(yr + seg * p.d + 8 * v) = pack8(o);
    }
    if (live && sub == 0) {
        p.mean[r] = mean;
        p.rstd[r] = rstd;
    }
}

template <int LPR, int VPL>
__global__ __launch_bounds__(256) void lmsd_bwd_kernel(LmsdParams p) {
    constexpr int RPW = 64 / LPR;
    __shared__ float red[4][2][8 * LPR * VPL];  // per wave: [dweight | dbias] of its vector slots
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int nvec = p.d / 8;
    const int64_t waves = (int64_t)gridDim.x * 4;
    const int64_t groups = (p.n + RPW - 1) / RPW;
    const int gseg = p.concat_u + p.concat_x;  // segment of l a in y and dy

    float w[VPL][8], bb[VPL][8];
    bool has[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = sub + k * LPR;
        has[k] = v < nvec;
        const int vv = has[k] ? v : 0;
        unpack8(ld_global16(p.weight + 8 * vv), w[k]);
        unpack8(ld_global16(p.bias + 8 * vv), bb[k]);
    }
    float accw[VPL][8], accb[VPL][8];
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) accw[k][i] = accb[k][i] = 0.0f;

    for (int64_t grp = (int64_t)blockIdx.x * 4 + wv; grp < groups; grp += waves) {
        const int64_t row = grp * RPW + lane / LPR;
        const bool live = row < p.n;
        const int64_t r = live ? row : p.n - 1;
        HSTU_DCHECK(r >= 0 && r < p.n, kDbgLmsd);
        const float mean = p.mean[r], rstd = p.rstd[r];
        const uint16_t* dyr = p.dy + r * p.dy_stride;
        float xh[VPL][8], a[VPL][8], g[VPL][8], dxh[VPL][8], uu[VPL][8];
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const int v = has[k] ? sub + k * LPR : 0;
            float x[8];
            unpack8(ld_global16(p.x + r * p.x_stride + 8 * v), x);
            unpack8(ld_global16(p.u + r * p.u_stride + 8 * v), uu[k]);
            unpack8(ld_global16(dyr + gseg * p.d + 8 * v), g[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xh[k][i] = (x[i] - mean) * rstd;
                a[k][i] = p.silu_u ? uu[k][i] * sigmoid(uu[k][i]) : uu[k][i];
                const float dl = live && has[k] ? g[k][i] * a[k][i] : 0.0f;
                dxh[k][i] = dl * w[k][i];
                s1 += dxh[k][i];
                s2 += dxh[k][i] * xh[k][i];
                accb[k][i] += dl;
                accw[k][i] += dl * xh[k][i];
            }
        }
        s1 = group_sum<LPR>(s1) * p.inv_d;
        s2 = group_sum<LPR>(s2) * p.inv_d;
        if (!live) continue;
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            if (!has[k]) continue;
            const int v = sub + k * LPR;
            float gu[8], gx[8], dx[8], du[8];
            if (p.concat_u) unpack8(ld_global16(dyr + 8 * v), gu);
            if (p.concat_x) unpack8(ld_global16(dyr + (p.concat_u ? p.d : 0) + 8 * v), gx);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                dx[i] = rstd * (dxh[k][i] - s1 - xh[k][i] * s2);
                if (p.concat_x) dx[i] += gx[i];
                float da = g[k][i] * (xh[k][i] * w[k][i] + bb[k][i]);
                if (p.concat_u) da += gu[i];
                if (p.silu_u) {
                    const float sg = sigmoid(uu[k][i]);
                    du[i] = da * sg * (1.0f + uu[k][i] * (1.0f - sg));
                } else {
                    du[i] = da;
                }
            }
            *reinterpret_cast<uint4*>(p.dx + r * p.dx_stride + 8 * v) = pack8(dx);
            *reinterpret_cast<uint4*>(p.du + r * p.du_stride + 8 * v) = pack8(du);
        }
    }

    // column partial sums: rows of the wave (lane groups) first, then the 4 waves
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) {
                accw[k][i] += __shfl_xor(accw[k][i], o, 64);
                accb[k][i] += __shfl_xor(accb[k][i], o, 64);
            }
    if (lane < LPR) {
#pragma unroll
        for (int k = 0; k < VPL; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                red[wv][0][(k * LPR + lane) * 8 + i] = accw[k][i];
                red[wv][1][(k * LPR + lane) * 8 + i] = accb[k][i];
            }
    }
    __syncthreads();
    // one partial row per workgroup: [dbias (D) | dweight (D) if computed]
    float* part = p.work + (int64_t)blockIdx.x * p.part_stride;
    // (vector slot k LPR + sub holds vector sub + k LPR, so column c sits at index c)
    for (int c = threadIdx.x; c < p.d; c += 256) {
        part[c] = red[0][1][c] + red[1][1][c] + red[2][1][c] + red[3][1][c];
        if (p.dweight) part[p.d + c] = red[0][0][c] + red[1][0][c] + red[2][0][c] + red[3][0][c];
    }
}

// dbias / dweight: column c of the partial rows (c < d: dbias, else dweight
// column c - d) is summed by one lane of each of the 16 waves of a workgroup --
// wave w takes the rows j = w (mod 16) in increasing order, eight loads in
// flight -- and the 16 wave sums are added in wave order through LDS.
__global__ __launch_bounds__(1024) void lmsd_colsum_kernel(LmsdParams p, int parts) {
    __shared__ float red[16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int pw = (int)p.part_stride;  // d, or 2 d with dweight
    float acc = 0.0f;
    if (c < pw) {
        int j = w;
        for (; j + 7 * 16 < parts; j += 8 * 16) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = p.work[(int64_t)(j + 16 * t) * pw + c];
#pragma unroll
            for (int t = 0; t < 8; ++t) acc += v[t];
        }
        for (; j < parts; j += 16) acc += p.work[(int64_t)j * pw + c];
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w != 0 || c >= pw) return;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += red[i][lane];
    const uint32_t h = pack_bf16x2(sum, 0.0f) & 0xffffu;
    if (c < p.d) p.dbias[c] = (uint16_t)h;
    else p.dweight[c - p.d] = (uint16_t)h;
}

template <int LPR, int VPL>
hipError_t launch_pair(const LmsdParams& p, bool bwd, int parts, hipStream_t stream) {
    if (!bwd) {
        constexpr int RPW = 64 / LPR;
        const int64_t waves = (p.n + RPW - 1) / RPW;
        hipLaunchKernelGGL((lmsd_fwd_kernel<LPR, VPL>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    if (parts > 0) {
        hipLaunchKernelGGL((lmsd_bwd_kernel<LPR, VPL>), dim3((unsigned)parts), dim3(256), 0, stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(lmsd_colsum_kernel, dim3((unsigned)((p.part_stride + 63) / 64)), dim3(1024), 0, stream, p,
                       parts);
    return hipGetLastError();
}

hipError_t launch(const LmsdParams& p, bool bwd, int parts, hipStream_t stream) {
    const int nvec = p.d / 8;
    if (nvec > 64) return launch_pair<64, 2>(p, bwd, parts, stream);
    if (nvec > 32) return launch_pair<64, 1>(p, bwd, parts, stream);
    if (nvec > 16) return launch_pair<32, 1>(p, bwd, parts, stream);
    if (nvec > 8) return launch_pair<16, 1>(p, bwd, parts, stream);
    if (nvec > 4) return launch_pair<8, 1>(p, bwd, parts, stream);
    if (nvec > 2) return launch_pair<4, 1>(p, bwd, parts, stream);
    if (nvec > 1) return launch_pair<2, 1>(p, bwd, parts, stream);
    return launch_pair<1, 1>(p, bwd, parts, stream);
}

}  // namespace

// Scratch for the column partials of hstu_lmsd_bwd_noalloc, for callers that
// cannot allocate: one array per GPU, held until the process ends and shared by
// every such call on that GPU.  It needs no clearing: each call's row kernel
// writes every partial row its column sums read.  Host code must not pass the
// array's name to a kernel (it is a host-side stand-in, not a device address):
// lmsd_scratch() returns the device's own address from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kLmsdScratchBytes / sizeof(float)];

hipError_t lmsd_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int lmsd_bwd_parts(int64_t n, int d) {
    const int nvec = d / 8;
    int lpr = 1;
    while (lpr < nvec && lpr < 64) lpr <<= 1;
    const int64_t groups = (n + 64 / lpr - 1) / (64 / lpr);
    const int64_t wgs = (groups + 3) / 4;
    return (int)(wgs < kLmsdMaxParts ? (wgs > 0 ? wgs : 1) : kLmsdMaxParts);
}

hipError_t launch_lmsd_fwd(const LmsdParams& p, hipStream_t stream) { return launch(p, false, 0, stream); }

#ifdef HSTU_DEBUG
hipError_t debug_take_lmsd(uint32_t* out) { return dbg_take(out); }
#endif

// parts = 0 (no rows) runs the column sums alone, which then write zeros.
hipError_t launch_lmsd_bwd(const LmsdParams& p, int parts, hipStream_t stream) { return launch(p, true, parts, stream); }

}  // namespace hstu
