// HSTU attention forward on gfx950.
//
// Computes, per packed sequence and head (HSTU Attention page, "Overview"
// equations), O = ((M (.) SiLU(alpha Q K^T)) / L_scale) V with no softmax, so no
// running maximum, no rescaling and no row statistics are kept: O is a plain
// sum over key tiles.
//
// Workgroup = 4 wavefronts = 128 query rows of one (sequence, head); each wave
// owns 32 rows.  Grid = (row block, sequence, head) flattened with the head
// fastest and the row block slowest in reverse, so the blocks with the most
// key tiles (the last rows of the longest causal sequences) start first.  A
// block past its sequence's end exits at once; the host never reads the
// cumulative lengths.
//
// Per key tile of 64 keys: K is staged row-major and V transposed in LDS
// (16-byte coalesced global loads; V is transposed in registers on the way in).
// Each wave then runs
//   S^T (64 x 32)  = K Q^T      on MFMA (A = K from LDS, B = Q from registers)
//   P^T            = bf16(S^T (.) sig(alpha S^T)), masked, in registers
//   O^T (D x 32)  += V^T P^T    on MFMA (A = V^T from LDS, B = P^T from registers)
// and the epilogue writes O = (alpha / L_scale) O^T^T in bf16.  Causal: only
// key tiles up to the block's last row are visited, and the per-element mask is
// applied only on tiles that cross the diagonal.  Key rows past the tile's end
// are staged as zeros, so they add exactly zero without a mask.
#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;  // 128 query rows per workgroup
constexpr int BN = 64;          // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;  // rows of the transposed V tile (32-row MFMA blocks)
    constexpr int D8 = D / 8;            // 16-byte groups per head-dim row
    constexpr int KSTR = D + 8;          // K tile row stride (elements); pad spreads banks
    constexpr int NCV = BN / 8;          // 16-byte column groups of a transposed row
    constexpr int VSTR = BN + 8;         // transposed V row stride (elements)
    constexpr int KSTEPS = D / 16;       // contraction steps of K Q^T
    constexpr int NSTEPS = BN / 16;      // contraction steps of V^T P^T

    __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt[DM * VSTR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    int idx = blockIdx.x;
    const int h = idx % p.heads;
    idx /= p.heads;
    const int b = idx % p.batch;
    const int m = p.nblk - 1 - idx / p.batch;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    const int m0 = m * BM;
    if (m0 >= sb.lq) return;

    const int kv_end = CAUSAL ? min(sb.lk, m0 + BM) : sb.lk;
    const int ntiles = (kv_end + BN - 1) / BN;

    const int row0 = m0 + 32 * wave;  // first (local) query row of this wave
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;

    uint4 qf[KSTEPS];
    if (my_row < sb.lq) {
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + my_row) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = ld_global16(src + 16 * kk);
    } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = make_uint4(0, 0, 0, 0);
    }

    if (DM > D) {  // padding rows of the transposed tile feed only discarded outputs; keep them finite
        for (int i = tid; i < (DM - D) * VSTR / 8; i += 256)
            st_lds16(vt + D * VSTR + 8 * i, make_uint4(0, 0, 0, 0));
    }

    f32x16 oacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) oacc[db] = f32x16{};

    const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
    const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;

    for (int t = 0; t < ntiles; ++t) {
        const int n0 = t * BN;
        __syncthreads();  // every wave is done reading the previous tile
        if (tid >= 128) {
            // K, row-major: consecutive threads take consecutive 16-byte groups of a row
            for (int c = tid - 128; c < BN * D8; c += 128) {
                const int r = c / D8, c8 = c % D8;
                uint4 val = make_uint4(0, 0, 0, 0);
                if (n0 + r < kv_end) val = ld_global16(kbase + (int64_t)(n0 + r) * p.k.tok + 8 * c8);
                st_lds16(ks + r * KSTR + 8 * c8, val);
            }
        } else {
            // V, transposed: a thread moves an 8 key x 8 dim block, keys in operand-slot order
            for (int bi = tid; bi < NCV * D8; bi += 128) {
                const int c8 = bi % D8, kg = bi / D8;
                uint4 in[8], out[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = n0 + group_row(kg, e);
                    in[e] = make_uint4(0, 0, 0, 0);
                    if (key < kv_end) in[e] = ld_global16(vbase + (int64_t)key * p.v.tok + 8 * c8);
                }
                transpose8x8(in, out);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = 8 * c8 + e;
                    st_lds16(vt + d * VSTR + 8 * swz<NCV>(kg, d), out[e]);
                }
            }
        }
        __syncthreads();

        if (!wave_live) continue;
        if (CAUSAL && n0 > row0 + 31) continue;  // every key of the tile is after every row of the wave

        f32x16 sacc[BN / 32];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                sacc[kb] = mfma32x32x16(ld_lds16(ks + (kb * 32 + l32) * KSTR + 16 * kk + 8 * g), qf[kk], sacc[kb]);
        }

        const bool diag = CAUSAL && (n0 + BN - 1 > row0);
        uint4 pf[NSTEPS];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = sacc[kb][r];
                float a = x * sigmoid_scaled(x, p.exp_c);
                if (diag) {
                    const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key > my_row) a = 0.0f;
                }
                pv[r] = a;
            }
            pf[2 * kb] = pack_operand(pv);
            pf[2 * kb + 1] = pack_operand(pv + 8);
        }

#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
            const int d = db * 32 + l32;
#pragma unroll
            for (int s = 0; s < NSTEPS; ++s)
                oacc[db] = mfma32x32x16(ld_lds16(vt + d * VSTR + 8 * swz<NCV>(2 * s + g, d)), pf[s], oacc[db]);
        }
    }

    if (my_row < sb.lq) {
        uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
        const float sc = p.out_scale;
#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = db * 32 + 8 * rq + 4 * g;
                if (d0 < D) {
                    const f32x16& a = oacc[db];
                    uint2 w = make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                         pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                    *reinterpret_cast<uint2*>(dst + d0) = w;
                }
            }
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.nblk * p.batch * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const AttnParams& p, int head_dim, bool causal, hipStream_t stream) {
    switch (head_dim) {
        case 16: return causal ? launch<16, true>(p, stream) : launch<16, false>(p, stream);
        case 32: return causal ? launch<32, true>(p, stream) : launch<32, false>(p, stream);
        case 64: return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
        case 128: return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hstu
