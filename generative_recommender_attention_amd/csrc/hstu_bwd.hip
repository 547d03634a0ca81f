// HSTU attention backward on gfx950: two deterministic kernels, no workspace.
//
// The backward receives dO and q, k, v only (HSTU Attention page, "High-level
// functions"), so both kernels recompute the scores.  With s = alpha q_i.k_j,
// a = SiLU(s) / L_scale and dA_ij = dO_i . v_j (chain rule on the page's
// "Overview" equations):
//     dV_j = sum_i M_ij a_ij dO_i
//     dQ_i = alpha sum_j M_ij dA_ij SiLU'(s_ij) / L_scale k_j
//     dK_j = alpha sum_i M_ij dA_ij SiLU'(s_ij) / L_scale q_i
// SiLU'(s) = sig(s) (1 + s (1 - sig(s))).  Both kernels carry x = q_i.k_j (no
// alpha) and fold alpha / L_scale into the final store, as the forward does.
//
// dq kernel: query-major, one workgroup per (128-row block, sequence, head), the
// same tile walk as the forward.  Per 64-key tile, K is staged row-major and
// transposed and V row-major; each wave computes S^T = K Q^T and dA^T = V dO^T,
// forms dS^T in registers and accumulates dQ^T += K^T dS^T.
//
// dk/dv kernel: key-major, one workgroup per (128-key block, sequence, head),
// each wave owning 32 keys held in registers.  Causal blocks walk query tiles
// from the block's first key to the end of the sequence (rows before it see
// none of these keys).  Per 64-row query tile, Q and dO are staged row-major and
// transposed; each wave computes S = Q K^T and dA = dO V^T, forms A' and dS in
// registers and accumulates dV^T += dO^T A' and dK^T += Q^T dS.
//
// Splitting the gradients over two kernels executes 14 D flops per visible pair
// against 10 D for a single pass, but needs no atomics and no dQ workspace and is
// bit-for-bit reproducible.
#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;  // dq kernel: query rows per workgroup (32 per wave)
constexpr int BN = 64;          // dq kernel: keys per tile
constexpr int BNK = kBwdBlockN; // dk/dv kernel: keys per workgroup (32 per wave)
constexpr int BMQ = 64;         // dk/dv kernel: query rows per tile

// SiLU'(alpha x) given sig = sig(alpha x).
__device__ __forceinline__ float dsilu(float x, float sig, float alpha) {
    return sig * (1.0f + alpha * x * (1.0f - sig));
}

// Stage one 8-row x 8-column block of a (rows, D) bf16 tile into LDS twice:
// row-major at rows group_row(c, e) and transposed at column group c.  Rows at
// or past `valid_end` (local) are zero.  `src` points at local row 0, column 0.
template <int D, int RSTR, int NC, int TSTR>
__device__ __forceinline__ void stage_block_both(const uint16_t* src, int64_t tok, int row_base, int valid_end,
                                                 int c, int c8, uint16_t* rm, uint16_t* tr) {
    uint4 in[8], out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int r = group_row(c, e);
        in[e] = make_uint4(0, 0, 0, 0);
        if (row_base + r < valid_end) in[e] = ld_global16(src + (int64_t)(row_base + r) * tok + 8 * c8);
        st_lds16(rm + r * RSTR + 8 * c8, in[e]);
    }
    transpose8x8(in, out);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = 8 * c8 + e;
        st_lds16(tr + d * TSTR + 8 * swz<NC>(c, d), out[e]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int D8 = D / 8;
    constexpr int KSTR = D + 8;
    constexpr int NCK = BN / 8;
    constexpr int TSTR = BN + 8;
    constexpr int KSTEPS = D / 16;
    constexpr int NSTEPS = BN / 16;

    __shared__ __attribute__((aligned(16))) uint16_t ks[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vs[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t kt[DM * TSTR];

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
    const int row0 = m0 + 32 * wave;
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;

    uint4 qf[KSTEPS], dof[KSTEPS];
    if (my_row < sb.lq) {
        const uint16_t* qs = p.q.base + (int64_t)(sb.q0 + my_row) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
        const uint16_t* ds = p.dout.base + (int64_t)(sb.q0 + my_row) * p.dout.tok + (int64_t)h * p.dout.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            qf[kk] = ld_global16(qs + 16 * kk);
            dof[kk] = ld_global16(ds + 16 * kk);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = dof[kk] = make_uint4(0, 0, 0, 0);
    }
    if (DM > D) {
        for (int i = tid; i < (DM - D) * TSTR / 8; i += 256)
            st_lds16(kt + D * TSTR + 8 * i, make_uint4(0, 0, 0, 0));
    }

    f32x16 dqacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) dqacc[db] = f32x16{};

    const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
    const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;

    for (int t = 0; t < ntiles; ++t) {
        const int n0 = t * BN;
        __syncthreads();
        if (tid < 128) {
            for (int bi = tid; bi < NCK * D8; bi += 128) {
                const int c8 = bi % D8, c = bi / D8;
                stage_block_both<D, KSTR, NCK, TSTR>(kbase, p.k.tok, n0, kv_end, c, c8, ks, kt);
            }
        } else {
            for (int c = tid - 128; c < BN * D8; c += 128) {
                const int r = c / D8, c8 = c % D8;
                uint4 val = make_uint4(0, 0, 0, 0);
                if (n0 + r < kv_end) val = ld_global16(vbase + (int64_t)(n0 + r) * p.v.tok + 8 * c8);
                st_lds16(vs + r * KSTR + 8 * c8, val);
            }
        }
        __syncthreads();

        if (!wave_live) continue;
        if (CAUSAL && n0 > row0 + 31) continue;

        f32x16 sacc[BN / 32], dacc[BN / 32];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            sacc[kb] = f32x16{};
            dacc[kb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int off = (kb * 32 + l32) * KSTR + 16 * kk + 8 * g;
                sacc[kb] = mfma32x32x16(ld_lds16(ks + off), qf[kk], sacc[kb]);
                dacc[kb] = mfma32x32x16(ld_lds16(vs + off), dof[kk], dacc[kb]);
            }
        }

        const bool diag = CAUSAL && (n0 + BN - 1 > row0);
        uint4 dsf[NSTEPS];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            float dv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = sacc[kb][r];
                const float sg = sigmoid_scaled(x, p.exp_c);
                float v = dacc[kb][r] * dsilu(x, sg, p.alpha);
                if (diag) {
                    const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key > my_row) v = 0.0f;
                }
                dv[r] = v;
            }
            dsf[2 * kb] = pack_operand(dv);
            dsf[2 * kb + 1] = pack_operand(dv + 8);
        }

#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
            const int d = db * 32 + l32;
#pragma unroll
            for (int s = 0; s < NSTEPS; ++s)
                dqacc[db] = mfma32x32x16(ld_lds16(kt + d * TSTR + 8 * swz<NCK>(2 * s + g, d)), dsf[s], dqacc[db]);
        }
    }

    if (my_row < sb.lq) {
        uint16_t* dst = p.dq.base + (int64_t)(sb.q0 + my_row) * p.dq.tok + (int64_t)h * p.dq.head;
        const float sc = p.out_scale;
#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = db * 32 + 8 * rq + 4 * g;
                if (d0 < D) {
                    const f32x16& a = dqacc[db];
                    *reinterpret_cast<uint2*>(dst + d0) =
                        make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                   pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                }
            }
        }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int D8 = D / 8;
    constexpr int QSTR = D + 8;
    constexpr int NCQ = BMQ / 8;
    constexpr int TSTR = BMQ + 8;
    constexpr int KSTEPS = D / 16;
    constexpr int NSTEPS = BMQ / 16;

    __shared__ __attribute__((aligned(16))) uint16_t qs[BMQ * QSTR];
    __shared__ __attribute__((aligned(16))) uint16_t dos[BMQ * QSTR];
    __shared__ __attribute__((aligned(16))) uint16_t qt[DM * TSTR];
    __shared__ __attribute__((aligned(16))) uint16_t dot[DM * TSTR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    // (key block n, sequence b, head h), key block 0 (the most query tiles) first
    int idx = blockIdx.x;
    const int h = idx % p.heads;
    idx /= p.heads;
    const int b = idx % p.batch;
    const int n = idx / p.batch;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    const int n0 = n * BNK;
    if (n0 >= sb.lk) return;

    const int key0 = n0 + 32 * wave;  // first (local) key of this wave
    const int my_key = key0 + l32;
    const bool wave_live = key0 < sb.lk;

    uint4 kf[KSTEPS], vf[KSTEPS];
    if (my_key < sb.lk) {
        const uint16_t* ks = p.k.base + (int64_t)(sb.k0 + my_key) * p.k.tok + (int64_t)h * p.k.head + 8 * g;
        const uint16_t* vs = p.v.base + (int64_t)(sb.k0 + my_key) * p.v.tok + (int64_t)h * p.v.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            kf[kk] = ld_global16(ks + 16 * kk);
            vf[kk] = ld_global16(vs + 16 * kk);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) kf[kk] = vf[kk] = make_uint4(0, 0, 0, 0);
    }
    if (DM > D) {
        for (int i = tid; i < (DM - D) * TSTR / 8; i += 256) {
            st_lds16(qt + D * TSTR + 8 * i, make_uint4(0, 0, 0, 0));
            st_lds16(dot + D * TSTR + 8 * i, make_uint4(0, 0, 0, 0));
        }
    }

    f32x16 dvacc[DM / 32], dkacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) dvacc[db] = dkacc[db] = f32x16{};

    const int q_begin = CAUSAL ? n0 : 0;  // causal: rows before the block's first key see none of it
    const int ntiles = sb.lq > q_begin ? (sb.lq - q_begin + BMQ - 1) / BMQ : 0;
    const uint16_t* qbase = p.q.base + (int64_t)sb.q0 * p.q.tok + (int64_t)h * p.q.head;
    const uint16_t* dbase = p.dout.base + (int64_t)sb.q0 * p.dout.tok + (int64_t)h * p.dout.head;

    for (int t = 0; t < ntiles; ++t) {
        const int qt0 = q_begin + t * BMQ;
        __syncthreads();
        if (tid < 128) {
            for (int bi = tid; bi < NCQ * D8; bi += 128) {
                const int c8 = bi % D8, c = bi / D8;
                stage_block_both<D, QSTR, NCQ, TSTR>(qbase, p.q.tok, qt0, sb.lq, c, c8, qs, qt);
            }
        } else {
            for (int bi = tid - 128; bi < NCQ * D8; bi += 128) {
                const int c8 = bi % D8, c = bi / D8;
                stage_block_both<D, QSTR, NCQ, TSTR>(dbase, p.dout.tok, qt0, sb.lq, c, c8, dos, dot);
            }
        }
        __syncthreads();

        if (!wave_live) continue;
        if (CAUSAL && qt0 + BMQ - 1 < key0) continue;  // every row of the tile precedes every key of the wave

        f32x16 sacc[BMQ / 32], dacc[BMQ / 32];
#pragma unroll
        for (int qb = 0; qb < BMQ / 32; ++qb) {
            sacc[qb] = f32x16{};
            dacc[qb] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int off = (qb * 32 + l32) * QSTR + 16 * kk + 8 * g;
                sacc[qb] = mfma32x32x16(ld_lds16(qs + off), kf[kk], sacc[qb]);
                dacc[qb] = mfma32x32x16(ld_lds16(dos + off), vf[kk], dacc[qb]);
            }
        }

        const bool diag = CAUSAL && (qt0 < key0 + 31);
        uint4 af[NSTEPS], dsf[NSTEPS];
#pragma unroll
        for (int qb = 0; qb < BMQ / 32; ++qb) {
            float av[16], dv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = sacc[qb][r];
                const float sg = sigmoid_scaled(x, p.exp_c);
                float a = x * sg;
                float d = dacc[qb][r] * dsilu(x, sg, p.alpha);
                if (diag) {
                    const int row = qt0 + qb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (my_key > row) a = d = 0.0f;
                }
                av[r] = a;
                dv[r] = d;
            }
            af[2 * qb] = pack_operand(av);
            af[2 * qb + 1] = pack_operand(av + 8);
            dsf[2 * qb] = pack_operand(dv);
            dsf[2 * qb + 1] = pack_operand(dv + 8);
        }

#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
            const int d = db * 32 + l32;
#pragma unroll
            for (int s = 0; s < NSTEPS; ++s) {
                const int off = d * TSTR + 8 * swz<NCQ>(2 * s + g, d);
                dvacc[db] = mfma32x32x16(ld_lds16(dot + off), af[s], dvacc[db]);
                dkacc[db] = mfma32x32x16(ld_lds16(qt + off), dsf[s], dkacc[db]);
            }
        }
    }

    if (my_key < sb.lk) {
        uint16_t* dk = p.dk.base + (int64_t)(sb.k0 + my_key) * p.dk.tok + (int64_t)h * p.dk.head;
        uint16_t* dv = p.dv.base + (int64_t)(sb.k0 + my_key) * p.dv.tok + (int64_t)h * p.dv.head;
        const float sc = p.out_scale;
#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = db * 32 + 8 * rq + 4 * g;
                if (d0 < D) {
                    const f32x16& a = dkacc[db];
                    const f32x16& c = dvacc[db];
                    *reinterpret_cast<uint2*>(dk + d0) =
                        make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                   pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                    *reinterpret_cast<uint2*>(dv + d0) =
                        make_uint2(pack_bf16x2(c[4 * rq] * sc, c[4 * rq + 1] * sc),
                                   pack_bf16x2(c[4 * rq + 2] * sc, c[4 * rq + 3] * sc));
                }
            }
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.nblk * p.batch * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.nblk * p.batch * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const AttnParams& p, int head_dim, bool causal, hipStream_t stream) {
    switch (head_dim) {
        case 16: return causal ? launch_dq<16, true>(p, stream) : launch_dq<16, false>(p, stream);
        case 32: return causal ? launch_dq<32, true>(p, stream) : launch_dq<32, false>(p, stream);
        case 64: return causal ? launch_dq<64, true>(p, stream) : launch_dq<64, false>(p, stream);
        case 128: return causal ? launch_dq<128, true>(p, stream) : launch_dq<128, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_dkdv(const AttnParams& p, int head_dim, bool causal, hipStream_t stream) {
    switch (head_dim) {
        case 16: return causal ? launch_dkdv<16, true>(p, stream) : launch_dkdv<16, false>(p, stream);
        case 32: return causal ? launch_dkdv<32, true>(p, stream) : launch_dkdv<32, false>(p, stream);
        case 64: return causal ? launch_dkdv<64, true>(p, stream) : launch_dkdv<64, false>(p, stream);
        case 128: return causal ? launch_dkdv<128, true>(p, stream) : launch_dkdv<128, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hstu
