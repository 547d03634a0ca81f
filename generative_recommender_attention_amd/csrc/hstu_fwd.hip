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
// Key tiles of 64 rows are staged row-major in swizzled LDS (one array: two K
// slots, two V slots) by direct global->LDS loads issued from inline assembly,
// double-buffered: the loads of tile t+1 are issued before tile t is computed,
// waited for (vmcnt) after it, and published by the one barrier per tile.  The
// compiler does not see those loads, so it adds no waits of its own and the
// LDS reads of the current tile are scheduled freely.  Reads use byte
// addresses whose slot, row-block and step parts fold into immediate offsets.
// Each wave runs
//   S^T (64 x 32)  = K (cQ)^T   on MFMA (A = K rows from LDS, B = Q from registers,
//                                scaled once by c = -alpha log2 e so the exponent is free)
//   P^T            = bf16(y / (1 + 2^y)), masked, in registers
//   O^T (D x 32)  += V^T P^T    on MFMA (A = V read transposed from LDS, B = P^T)
// with every LDS read issued a few products ahead of its MFMA, P^T of the
// first 32 keys computed while the second block's products run, and the
// epilogue writing O = (alpha / L_scale) O^T^T in bf16.  Causal: only key tiles
// up to the block's last row are visited, waves skip tiles entirely after
// their rows, and the per-element mask runs only on tiles that cross the
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
        keep_branch();
#pragma unroll
        for (int r = 0; r < 8; ++r) pv[r] = key0 + acc_row(r0 + r, g) < lim ? pv[r] : 0.0f;
    }
    return pack_operand(pv);
}

constexpr uint32_t kTileBytes = 2 * kTileElems;  // 16 KB per staged 64-row tile

// One key tile for one wave.  S^T for the first 32 keys (s0), then for the second
// 32 (s1), each one accumulation chain; K rows are read PF steps ahead of the
// MFMA that uses them.  P^T of s0 is computed while s1's products run, and the
// first half of O^T += V^T P^T runs while P^T of s1 is computed.
template <int D>
__device__ __forceinline__ void fwd_tile(uint32_t kt, uint32_t vt, const uint4 (&qf)[D / 16],
                                            f32x16 (&oacc)[(D < 32 ? 32 : D) / 32], const uint32_t (&koff)[D / 16],
                                            const uint2 (&voff)[(D < 32 ? 32 : D) / 32], int n0, int lim, int wlim,
                                            int g) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;
    constexpr int NS = D / 16;  // contraction steps per key block
    constexpr int NK = 2 * NS;  // K reads: block-major, step-minor
    constexpr int NO = 4 * NDB; // V reads / O products: step-major, column-block-minor
    constexpr int PF = 4;
    // one read per product, issued in product order: r < NK reads K for S, r >= NK reads V for O
    uint4 rd[NK + NO];
    auto read = [&](int r) {
        if (r < NK) {
            rd[r] = ds_read16(koff[r % NS] + kt + (r / NS) * 8192);
        } else if (r < NK + NO) {
            const int s4 = (r - NK) / NDB, db = (r - NK) % NDB;
            rd[r] = ds_read_tr16x2(voff[db].x + vt + 4096 * s4, voff[db].y + vt + 4096 * s4);
        }
    };
#pragma unroll
    for (int r = 0; r < PF; ++r) read(r);
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        if (j < NS) s0 = mfma32x32x16(rd[j], qf[j], s0);
        else s1 = mfma32x32x16(rd[j], qf[j - NS], s1);
        read(j + PF);
    }
    const uint4 p0 = fwd_scores_op(s0, 0, n0, lim, wlim, g);
    const uint4 p1 = fwd_scores_op(s0, 8, n0, lim, wlim, g);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < NDB ? p0 : p1, oacc[i % NDB]);
        read(NK + i + PF);
    }
    const uint4 p2 = fwd_scores_op(s1, 0, n0 + 32, lim, wlim, g);
    const uint4 p3 = fwd_scores_op(s1, 8, n0 + 32, lim, wlim, g);
#pragma unroll
    for (int i = 2 * NDB; i < NO; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < 3 * NDB ? p2 : p3, oacc[i % NDB]);
        read(NK + i + PF);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int KSTEPS = D / 16;
    // [K slot 0 | K slot 1 | V slot 0 | V slot 1]; tile t lives in slot t % 2
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTileElems];
    const uint32_t lds0 = lds_addr(smem);
    constexpr uint32_t K0 = 0, K1 = kTileBytes, V0 = 2 * kTileBytes, V1 = 3 * kTileBytes;

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
    const int wlim = CAUSAL ? min(kv_end, row0 + 1) : kv_end;

    uint4 qf[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = scale_bf16x8(ld_global16(src + 16 * kk), p.exp_c);
    }
    uint32_t koff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = lds0 + tile_byte(l32, 2 * kk + g);
    uint2 voff[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        voff[db] = tr_offsets(32 * db, lane);
        voff[db].x += lds0;
        voff[db].y += lds0;
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
        if constexpr (D < 32) {
            // columns D..31 of every slot are read by the 32-wide MFMA blocks
            for (int u = tid; u < 4 * kTileRows * (32 - D) / 8; u += 256) {
                const int sl = u / (kTileRows * (32 - D) / 8), v = u % (kTileRows * (32 - D) / 8);
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        kdma.issue(lds0 + K0, kbase, p.k.tok, 0, kv_end);
        vdma.issue(lds0 + V0, vbase, p.v.tok, 0, kv_end);
        wait_global_loads();
        __syncthreads();

        auto step = [&](uint32_t kc, uint32_t vc, uint32_t kn, uint32_t vn, int t) {
            const int n0 = t * BN;
            if (t + 1 < ntiles) {  // the other slots were last read before the previous barrier
                kdma.issue(lds0 + kn, kbase, p.k.tok, n0 + BN, kv_end);
                vdma.issue(lds0 + vn, vbase, p.v.tok, n0 + BN, kv_end);
            }
            // waves whose rows all precede the tile's first key, or lie past the sequence, skip it
            if (wave_live && !(CAUSAL && n0 > row0 + 31)) fwd_tile<D>(kc, vc, qf, oacc, koff, voff, n0, lim, wlim, g);
            wait_global_loads();
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(K0, V0, K1, V1, t);
            if (t + 1 < ntiles) step(K1, V1, K0, V0, t + 1);
        }
    }

    if (my_row < sb.lq) {
        uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
        const float sc = p.pre_scale;
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
