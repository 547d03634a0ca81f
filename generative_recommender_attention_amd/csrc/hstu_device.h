// Device-side building blocks shared by the HSTU attention kernels (gfx950).
//
// Matrix products run on the CDNA4 instruction v_mfma_f32_32x32x16_bf16
// (a 32x32 fp32 tile += 32x16 bf16 * 16x32 bf16, one wavefront of 64 lanes).
// Operand and accumulator placement used throughout, for lane l = 0..63,
// l32 = l % 32 and g = l / 32:
//   A (32 rows x 16 k):  lane holds row l32, k = 8g .. 8g+7   (one 16-byte value)
//   B (16 k x 32 cols):  lane holds col l32, k = 8g .. 8g+7   (one 16-byte value)
//   C (32 x 32, fp32):   lane holds col l32, rows 8(r/4) + 4g + r%4, r = 0..15
// An accumulator C[m][n] therefore keeps its column index in the lane and its
// row index in the register.  The kernels exploit that: the fp32 tile of one
// product, rounded to bf16 in registers, is directly the B operand of the next
// product that contracts over C's row index, with no trip through LDS.  The
// order of the 16 contraction slots is free as long as both operands agree; the
// B operand built from an accumulator takes, for contraction step s (16 rows of
// C), slot t <- row 16s + 4g + (t%4) + 8(t/4), i.e. registers 8(s%2)+t of the
// 32-row block s/2.  The A operand for such a product is read from a transposed
// LDS tile whose 16-byte column groups hold the same rows in the same order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// One (T, H, D) bf16 tensor: element (t, h, d) at base + t*tok + h*head + d.
struct TensorRef {
    const uint16_t* base;
    int64_t tok;
    int64_t head;
};
struct TensorOut {
    uint16_t* base;
    int64_t tok;
    int64_t head;
};

__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Round two fp32 values to bf16 (nearest-even, v_cvt_pk_bf16_f32) and pack
// them into one dword, `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf16 B operand from registers r0..r0+7 of an fp32 accumulator-shaped array.
__device__ __forceinline__ uint4 pack_operand(const float* x) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 ld_lds16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st_lds16(uint16_t* p, uint4 v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// 8 x 8 transpose of bf16 held as eight 16-byte rows: out[e] element t =
// in[t] element e.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t w[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t* a = reinterpret_cast<const uint32_t*>(&in[2 * c]);
            const uint32_t* b = reinterpret_cast<const uint32_t*>(&in[2 * c + 1]);
            const uint32_t x = a[e >> 1], y = b[e >> 1];
            w[c] = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        }
        out[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Row (within a tile) of element t of 16-byte column group c of a transposed
// tile: the contraction-slot order of an accumulator-built B operand.
__device__ __forceinline__ int group_row(int c, int t) {
    return 16 * (c >> 1) + 4 * (c & 1) + (t & 3) + 8 * (t >> 2);
}

// Transposed tiles: row d (a head-dim index) of NC 16-byte column groups, with
// the group index XOR-swizzled by d/8 so that both the staging writes (eight
// lanes = eight consecutive d/8 at one group) and the MFMA reads (eight lanes =
// eight consecutive d at one group) spread over all LDS banks.
template <int NC>
__device__ __forceinline__ int swz(int c, int d) {
    return c ^ ((d >> 3) & (NC - 1));
}

// Sequence bounds of batch entry b.
struct SeqBounds {
    int q0, lq, k0, lk;
};
__device__ __forceinline__ SeqBounds seq_bounds(const int32_t* cu_q, const int32_t* cu_k, int b) {
    SeqBounds s;
    s.q0 = cu_q[b];
    s.lq = cu_q[b + 1] - s.q0;
    s.k0 = cu_k[b];
    s.lk = cu_k[b + 1] - s.k0;
    return s;
}

// SiLU(alpha x) / alpha = x * sig(alpha x), with sig(y) = 1 / (1 + 2^(-y log2 e)).
// `c` = -alpha * log2(e).  v_exp_f32 and v_rcp_f32 (about 1 ulp each); large
// |x| saturate cleanly: 2^+big = inf -> rcp = 0, 2^-big = 0 -> rcp = 1.
__device__ __forceinline__ float sigmoid_scaled(float x, float c) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * c));
}

}  // namespace hstu
