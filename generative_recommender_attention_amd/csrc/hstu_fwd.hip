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
// Key tiles of 64 rows are staged row-major in swizzled LDS by direct
// global->LDS loads, double-buffered: the loads of tile t+1 are issued before
// tile t is computed, so their latency hides behind it and one barrier per
// tile suffices.  Each wave runs
//   S^T (64 x 32)  = K (cQ)^T   on MFMA (A = K rows from LDS, B = Q from registers,
//                                scaled once by c = -alpha log2 e so the exponent is free)
//   P^T            = bf16(y / (1 + 2^y)), masked, in registers
//   O^T (D x 32)  += V^T P^T    on MFMA (A = V read transposed from LDS, B = P^T)
// and the epilogue writes O = (alpha / L_scale) O^T^T in bf16.  Causal: only
// key tiles up to the block's last row are visited, waves skip tiles entirely
// after their rows, and the per-element mask runs only on tiles that cross the
// diagonal or the sequence end.
#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;  // 128 query rows per workgroup, 32 per wave
constexpr int BN = kTileRows;   // 64 keys per tile

// bf16 P^T operand from accumulator registers r0..r0+7.  The scores arrive as
// y = c x with c = -alpha log2(e) folded into Q (x = q.k), so
// y sig(alpha x) = y / (1 + 2^y) costs one exp, one add, one rcp and one
// multiply; the factor 1/c is folded into the output scale.  Keys at or past
// `lim` are zeroed; only blocks reaching `wlim` (the smallest `lim` of the
// wave) pay for the selects.
__device__ __forceinline__ uint4 fwd_scores_op(const f32x16& sacc, int r0, int key0, int lim, int wlim, int g) {
    float pv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pv[r] = silu_pre(sacc[r0 + r]);
    if (key0 + 32 > wlim) {
#pragma unroll
        for (int r = 0; r < 8; ++r) pv[r] = key0 + acc_row(r0 + r, g) < lim ? pv[r] : 0.0f;
    }
    return pack_operand(pv);
}

// One key tile for one wave: S^T = K Q^T for both 32-key blocks (two
// independent MFMA chains), then per block P^T = bf16(y sig(alpha x)) masked to
// keys below `lim` and O^T += V^T P^T.
template <int D>
__device__ __forceinline__ void fwd_tile(const uint16_t* ks, const uint16_t* vs, const uint4 (&qf)[D / 16],
                                         f32x16 (&oacc)[(D < 32 ? 32 : D) / 32], int n0, int lim, int wlim,
                                         int lane) {
    constexpr int DM = D < 32 ? 32 : D;
    const int l32 = lane & 31, g = lane >> 5;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) s0 = mfma32x32x16(lds_read16(ks, l32, 16 * kk + 8 * g), qf[kk], s0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) s1 = mfma32x32x16(lds_read16(ks, 32 + l32, 16 * kk + 8 * g), qf[kk], s1);
    const uint4 p0 = fwd_scores_op(s0, 0, n0, lim, wlim, g);
    const uint4 p1 = fwd_scores_op(s0, 8, n0, lim, wlim, g);
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        oacc[db] = mfma32x32x16(lds_read_transposed(vs, 0, db * 32, lane), p0, oacc[db]);
        oacc[db] = mfma32x32x16(lds_read_transposed(vs, 1, db * 32, lane), p1, oacc[db]);
    }
    const uint4 p2 = fwd_scores_op(s1, 0, n0 + 32, lim, wlim, g);
    const uint4 p3 = fwd_scores_op(s1, 8, n0 + 32, lim, wlim, g);
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        oacc[db] = mfma32x32x16(lds_read_transposed(vs, 2, db * 32, lane), p2, oacc[db]);
        oacc[db] = mfma32x32x16(lds_read_transposed(vs, 3, db * 32, lane), p3, oacc[db]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;  // rows of the O^T accumulator (32-row MFMA blocks)
    constexpr int KSTEPS = D / 16;       // contraction steps of K Q^T

    // two separate buffers per operand, so the compiler can tell the tile being
    // read from the tile being filled and need not wait for the fill
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

    const int row0 = m0 + 32 * wave;  // first (local) query row of this wave
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;
    // keys at or past `lim` contribute nothing to this lane's row
    const int lim = CAUSAL ? min(kv_end, my_row + 1) : kv_end;
    const int wlim = CAUSAL ? min(kv_end, row0 + 1) : kv_end;  // smallest lim in the wave

    uint4 qf[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = scale_bf16x8(ld_global16(src + 16 * kk), p.exp_c);
    }

    f32x16 oacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) oacc[db] = f32x16{};

    if (ntiles > 0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D> kdma, vdma;
        kdma.init(wave, lane, p.k.tok);
        vdma.init(wave, lane, p.v.tok);
        zero_tile_tail<D>(ks0, tid);
        zero_tile_tail<D>(ks1, tid);
        zero_tile_tail<D>(vs0, tid);
        zero_tile_tail<D>(vs1, tid);
        kdma.issue(ks0, kbase, p.k.tok, 0, kv_end);
        vdma.issue(vs0, vbase, p.v.tok, 0, kv_end);
        wait_global_loads();
        __syncthreads();

        auto step = [&](const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn, int t) {
            const int n0 = t * BN;
            if (t + 1 < ntiles) {  // the other buffers were last read before the previous barrier
                kdma.issue(kn, kbase, p.k.tok, n0 + BN, kv_end);
                vdma.issue(vn, vbase, p.v.tok, n0 + BN, kv_end);
            }
            // waves whose rows all precede the tile's first key, or lie past the sequence, skip it
            if (wave_live && !(CAUSAL && n0 > row0 + 31)) fwd_tile<D>(kc, vc, qf, oacc, n0, lim, wlim, lane);
            wait_global_loads();
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(ks0, vs0, ks1, vs1, t);
            if (t + 1 < ntiles) step(ks1, vs1, ks0, vs0, t + 1);
        }
    }

    if (my_row < sb.lq) {
        uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
        const float sc = p.pre_scale;  // alpha / L_scale, and undo the c folded into the scores
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
