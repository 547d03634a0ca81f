// HSTU attention backward on gfx950: two deterministic kernels, no workspace.
//
// The backward receives dO and q, k, v only (HSTU Attention page, "High-level
// functions"), so both kernels recompute the scores.  With s = alpha q_i.k_j,
// a = SiLU(s) / L_scale and dA_ij = dO_i . v_j (chain rule on the page's
// "Overview" equations):
//     dV_j = sum_i M_ij a_ij dO_i
//     dQ_i = alpha sum_j M_ij dA_ij SiLU'(s_ij) / L_scale k_j
//     dK_j = alpha sum_i M_ij dA_ij SiLU'(s_ij) / L_scale q_i
// SiLU'(s) = sig(s) (1 + s (1 - sig(s))).  As in the forward, the score MFMAs
// run on Q (dq kernel) or K (dk/dv kernel) pre-multiplied by c = -alpha log2 e,
// so they produce y = c x (x = q_i.k_j): sig(s) = 1 / (1 + 2^y) and
// s = alpha x = -y / log2 e; alpha / L_scale (and 1/c for dV) is applied at the
// final store.
//
// dq kernel: query-major, one workgroup per (128-row block, sequence, head), the
// same tile walk as the forward.  Per 64-key tile K and V are staged row-major
// in LDS; each wave computes S^T = K Q^T and dA^T = V dO^T (A operands: K, V
// rows), forms dS^T in registers and accumulates dQ^T += K^T dS^T (A operand:
// K read transposed).
//
// dk/dv kernel: key-major, one workgroup per (128-key block, sequence, head),
// each wave owning 32 keys held in registers.  Causal blocks walk query tiles
// from the block's first key to the end of the sequence (rows before it see
// none of these keys).  Per 64-row query tile Q and dO are staged row-major;
// each wave computes S = Q K^T and dA = dO V^T (A operands: Q, dO rows), forms
// A' and dS in registers and accumulates dV^T += dO^T A' and dK^T += Q^T dS
// (A operands: dO, Q read transposed).
//
// Tiles are staged by direct global->LDS loads into two buffers per operand:
// tile t+1 loads while tile t is computed.  Splitting the gradients over two
// kernels executes 14 D flops per visible pair against 10 D for a single pass,
// but needs no atomics and no workspace and is bit-for-bit reproducible.
#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;   // dq kernel: query rows per workgroup (32 per wave)
constexpr int BN = kTileRows;    // dq kernel: keys per tile
constexpr int BNK = kBwdBlockN;  // dk/dv kernel: keys per workgroup (32 per wave)
constexpr int BMQ = kTileRows;   // dk/dv kernel: query rows per tile

constexpr float kNegLn2 = -0.69314718055994531f;  // s = y * kNegLn2 for y = c x

// sig(s) and SiLU'(s) = sig (1 + s (1 - sig)) from a pre-scaled score y.
__device__ __forceinline__ float sig_pre(float y) { return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y)); }
__device__ __forceinline__ float dsilu_pre(float y, float sig) {
    return sig * __builtin_fmaf(y * kNegLn2, 1.0f - sig, 1.0f);
}

// One key tile of the dq kernel for one wave.
template <int D>
__device__ __forceinline__ void dq_tile(const uint16_t* ks, const uint16_t* vs, const uint4 (&qf)[D / 16],
                                        const uint4 (&dof)[D / 16], f32x16 (&acc)[(D < 32 ? 32 : D) / 32], int n0,
                                        int lim, int wlim, int lane) {
    constexpr int DM = D < 32 ? 32 : D;
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
        f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            sacc = mfma32x32x16(lds_read16(ks, kb * 32 + l32, 16 * kk + 8 * g), qf[kk], sacc);
            dacc = mfma32x32x16(lds_read16(vs, kb * 32 + l32, 16 * kk + 8 * g), dof[kk], dacc);
        }
        float dv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[r] = dacc[r] * dsilu_pre(sacc[r], sig_pre(sacc[r]));
        if (n0 + kb * 32 + 32 > wlim) {  // only blocks crossing the mask pay for the selects
            keep_branch();
#pragma unroll
            for (int r = 0; r < 16; ++r) dv[r] = n0 + kb * 32 + acc_row(r, g) < lim ? dv[r] : 0.0f;
        }
        const uint4 d0 = pack_operand(dv), d1 = pack_operand(dv + 8);
#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
            acc[db] = mfma32x32x16(lds_read_transposed(ks, 2 * kb, db * 32, lane), d0, acc[db]);
            acc[db] = mfma32x32x16(lds_read_transposed(ks, 2 * kb + 1, db * 32, lane), d1, acc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int KSTEPS = D / 16;

    __shared__ __attribute__((aligned(16))) uint16_t ks0[kTileElems], ks1[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t vs0[kTileElems], vs1[kTileElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

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
    const int lim = CAUSAL ? min(kv_end, my_row + 1) : kv_end;
    const int wlim = CAUSAL ? min(kv_end, row0 + 1) : kv_end;  // smallest lim in the wave

    uint4 qf[KSTEPS], dof[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        const uint16_t* qsrc = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
        const uint16_t* dsrc = p.dout.base + (int64_t)(sb.q0 + r) * p.dout.tok + (int64_t)h * p.dout.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            qf[kk] = scale_bf16x8(ld_global16(qsrc + 16 * kk), p.exp_c);  // fold c into Q
            dof[kk] = ld_global16(dsrc + 16 * kk);
        }
    }

    f32x16 acc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) acc[db] = f32x16{};

    if (ntiles > 0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D> kdma, vdma;
        kdma.init(wave, lane, p.k.tok);
        vdma.init(wave, lane, p.v.tok);
        zero_tile_tail<D>(ks0, tid);
        zero_tile_tail<D>(ks1, tid);
        kdma.issue(ks0, kbase, p.k.tok, 0, kv_end);
        vdma.issue(vs0, vbase, p.v.tok, 0, kv_end);
        wait_global_loads();
        __syncthreads();

        auto step = [&](const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn, int t) {
            const int n0 = t * BN;
            if (t + 1 < ntiles) {
                kdma.issue(kn, kbase, p.k.tok, n0 + BN, kv_end);
                vdma.issue(vn, vbase, p.v.tok, n0 + BN, kv_end);
            }
            if (wave_live && !(CAUSAL && n0 > row0 + 31))
                dq_tile<D>(kc, vc, qf, dof, acc, n0, lim, wlim, lane);
            wait_global_loads();
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(ks0, vs0, ks1, vs1, t);
            if (t + 1 < ntiles) step(ks1, vs1, ks0, vs0, t + 1);
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
                    const f32x16& a = acc[db];
                    *reinterpret_cast<uint2*>(dst + d0) =
                        make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                   pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                }
            }
        }
    }
}

// One query tile of the dk/dv kernel for one wave; rows outside [lo, hi) are
// masked (lo is per lane); only blocks with rows below `wlo` (the largest lo of
// the wave) or at or past hi pay for the selects.
template <int D>
__device__ __forceinline__ void dkdv_tile(const uint16_t* qs, const uint16_t* dos, const uint4 (&kf)[D / 16],
                                          const uint4 (&vf)[D / 16], f32x16 (&dvacc)[(D < 32 ? 32 : D) / 32],
                                          f32x16 (&dkacc)[(D < 32 ? 32 : D) / 32], int qt0, int lo, int wlo,
                                          int hi, int lane) {
    constexpr int DM = D < 32 ? 32 : D;
    const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
        f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            sacc = mfma32x32x16(lds_read16(qs, qb * 32 + l32, 16 * kk + 8 * g), kf[kk], sacc);
            dacc = mfma32x32x16(lds_read16(dos, qb * 32 + l32, 16 * kk + 8 * g), vf[kk], dacc);
        }
        float av[16], dv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float y = sacc[r], sg = sig_pre(y);
            av[r] = y * sg;
            dv[r] = dacc[r] * dsilu_pre(y, sg);
        }
        const int row0 = qt0 + qb * 32;
        if (row0 < wlo || row0 + 32 > hi) {
            keep_branch();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + acc_row(r, g);
                const bool ok = row >= lo && row < hi;
                av[r] = ok ? av[r] : 0.0f;
                dv[r] = ok ? dv[r] : 0.0f;
            }
        }
        const uint4 a0 = pack_operand(av), a1 = pack_operand(av + 8);
        const uint4 d0 = pack_operand(dv), d1 = pack_operand(dv + 8);
#pragma unroll
        for (int db = 0; db < DM / 32; ++db) {
            dvacc[db] = mfma32x32x16(lds_read_transposed(dos, 2 * qb, db * 32, lane), a0, dvacc[db]);
            dvacc[db] = mfma32x32x16(lds_read_transposed(dos, 2 * qb + 1, db * 32, lane), a1, dvacc[db]);
            dkacc[db] = mfma32x32x16(lds_read_transposed(qs, 2 * qb, db * 32, lane), d0, dkacc[db]);
            dkacc[db] = mfma32x32x16(lds_read_transposed(qs, 2 * qb + 1, db * 32, lane), d1, dkacc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int KSTEPS = D / 16;

    __shared__ __attribute__((aligned(16))) uint16_t qs0[kTileElems], qs1[kTileElems];
    __shared__ __attribute__((aligned(16))) uint16_t ds0[kTileElems], ds1[kTileElems];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

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
    {
        const int r = min(my_key, sb.lk - 1);
        const uint16_t* ksrc = p.k.base + (int64_t)(sb.k0 + r) * p.k.tok + (int64_t)h * p.k.head + 8 * g;
        const uint16_t* vsrc = p.v.base + (int64_t)(sb.k0 + r) * p.v.tok + (int64_t)h * p.v.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            kf[kk] = scale_bf16x8(ld_global16(ksrc + 16 * kk), p.exp_c);  // fold c into K
            vf[kk] = ld_global16(vsrc + 16 * kk);
        }
    }

    f32x16 dvacc[DM / 32], dkacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) dvacc[db] = dkacc[db] = f32x16{};

    const int q_begin = CAUSAL ? n0 : 0;  // causal: rows before the block's first key see none of it
    const int ntiles = sb.lq > q_begin ? (sb.lq - q_begin + BMQ - 1) / BMQ : 0;
    // rows this lane's key is visible to: [lo, sb.lq)
    const int lo = CAUSAL ? my_key : 0;
    const int wlo = CAUSAL ? key0 + 31 : 0;  // largest lo in the wave

    if (ntiles > 0) {
        const uint16_t* qbase = p.q.base + (int64_t)sb.q0 * p.q.tok + (int64_t)h * p.q.head;
        const uint16_t* dbase = p.dout.base + (int64_t)sb.q0 * p.dout.tok + (int64_t)h * p.dout.head;
        TileDma<D> qdma, ddma;
        qdma.init(wave, lane, p.q.tok);
        ddma.init(wave, lane, p.dout.tok);
        zero_tile_tail<D>(qs0, tid);
        zero_tile_tail<D>(qs1, tid);
        zero_tile_tail<D>(ds0, tid);
        zero_tile_tail<D>(ds1, tid);
        qdma.issue(qs0, qbase, p.q.tok, q_begin, sb.lq);
        ddma.issue(ds0, dbase, p.dout.tok, q_begin, sb.lq);
        wait_global_loads();
        __syncthreads();

        auto step = [&](const uint16_t* qc, const uint16_t* dc, uint16_t* qn, uint16_t* dn, int t) {
            const int qt0 = q_begin + t * BMQ;
            if (t + 1 < ntiles) {
                qdma.issue(qn, qbase, p.q.tok, qt0 + BMQ, sb.lq);
                ddma.issue(dn, dbase, p.dout.tok, qt0 + BMQ, sb.lq);
            }
            // waves whose keys all follow every row of the tile, or lie past the sequence, skip it
            if (wave_live && !(CAUSAL && qt0 + BMQ - 1 < key0))
                dkdv_tile<D>(qc, dc, kf, vf, dvacc, dkacc, qt0, lo, wlo, sb.lq, lane);
            wait_global_loads();
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(qs0, ds0, qs1, ds1, t);
            if (t + 1 < ntiles) step(qs1, ds1, qs0, ds0, t + 1);
        }
    }

    if (my_key < sb.lk) {
        uint16_t* dk = p.dk.base + (int64_t)(sb.k0 + my_key) * p.dk.tok + (int64_t)h * p.dk.head;
        uint16_t* dv = p.dv.base + (int64_t)(sb.k0 + my_key) * p.dv.tok + (int64_t)h * p.dv.head;
        const float sc = p.out_scale, scv = p.pre_scale;
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
                        make_uint2(pack_bf16x2(c[4 * rq] * scv, c[4 * rq + 1] * scv),
                                   pack_bf16x2(c[4 * rq + 2] * scv, c[4 * rq + 3] * scv));
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
