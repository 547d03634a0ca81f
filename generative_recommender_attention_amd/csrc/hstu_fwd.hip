// HSTU attention forward on gfx950.
//
// Computes, per packed sequence and head (HSTU Attention page, "Overview"
// equations), O = ((M (.) SiLU(alpha Q K^T)) / L_scale) V with no softmax, so no
// running maximum, no rescaling and no row statistics are kept: O is a plain
// sum over key tiles, and any split of the keys combines by addition.
//
// Workgroup = 4 wavefronts on the 4 SIMDs of one CU (one workgroup per CU, so
// each wave may use the full 512-register file) = 128 query rows of one
// (sequence, head).  Wave w owns the 64 rows 64 (w & 1) .. +63 and the key
// tiles of parity w >> 1: the two wave pairs run the even and the odd 64-key
// tiles of the same rows, which halves the longest chain of tiles a workgroup
// walks (the last rows of a long causal sequence), and add their partial O
// through LDS at the end.  Grid = (row block, sequence, head) flattened with
// the head fastest and the row block slowest in reverse, so the blocks with the
// most key tiles start first.  A block past its sequence's end exits at once;
// the host never reads the cumulative lengths.
//
// Each wave pair stages its own tiles (64 keys x D of K and of V, row-major,
// swizzled) into LDS with direct global->LDS loads issued from inline assembly,
// double-buffered: the loads of the pair's next tile are issued before the
// current one is computed and waited for (vmcnt) before the one barrier per
// step.  Per tile a wave runs, for each 32-key half,
//   S^T (32 x 64)  = K_half (cQ)^T   on MFMA: A = K rows from LDS, B = Q from
//                    registers (64 rows = two 32-row blocks, so every LDS read
//                    feeds two MFMAs), Q pre-scaled by c = -alpha log2 e
//   P^T            = bf16(y / (1 + 2^y)), masked on edge tiles only
//   O^T (D x 64)  += V_half^T P^T    on MFMA: A = V read transposed from LDS
// with the scores of one half turned into P^T while the next half's products
// run, and the epilogue writing O = (alpha / L_scale) O^T^T in bf16.
#include <type_traits>

#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;                   // 128 query rows per workgroup
constexpr int BN = kTileRows;                    // 64 keys per tile
constexpr uint32_t kTileBytes = 2 * kTileElems;  // 16 KB per staged 64-row tile
constexpr uint32_t kGroupBytes = 4 * kTileBytes; // per wave pair: K slots 0, 1, V slots 0, 1

// bf16 P^T operand from accumulator registers r0..r0+7 of a 32-key block whose
// first key is key0.  The scores arrive as y = c x with c = -alpha log2(e)
// folded into Q (x = q.k), so y sig(alpha x) = y / (1 + 2^y) costs one exp, one
// add, one rcp and one multiply; the factor 1/c is folded into the output
// scale.  With MASKED, keys at or past this lane's limit `lim` are zeroed.
template <bool MASKED>
__device__ __forceinline__ uint4 silu_operand(const f32x16& s, int r0, int key0, int lim, int g) {
    float pv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pv[r] = silu_pre(s[r0 + r]);
    if constexpr (MASKED) {
#pragma unroll
        for (int r = 0; r < 8; ++r) pv[r] = key0 + acc_row(r0 + r, g) < lim ? pv[r] : 0.0f;
    }
    return pack_operand(pv);
}

// One 64-key tile for one wave of 64 query rows (two 32-row blocks rb).
// Reads are issued in product order, PF reads ahead of the MFMAs that use them;
// each read feeds the two row blocks' products.
template <int D, bool MASKED>
__device__ __forceinline__ void fwd_tile(uint32_t kt, uint32_t vt, const uint4 (&qf)[2][D / 16],
                                         f32x16 (&oacc)[(D < 32 ? 32 : D) / 32][2], const uint32_t (&koff)[D / 16],
                                         const uint2 (&voff)[(D < 32 ? 32 : D) / 32], int n0, const int (&lim)[2],
                                         int g) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;  // 32-column blocks of O^T
    constexpr int NS = D / 16;                   // contraction steps per S^T block
    constexpr int NK = 2 * NS;                   // K reads: half-major, step-minor
    constexpr int NV = 4 * NDB;                  // V reads: key step-major, column block-minor
    constexpr int PF = 4;
    uint4 rd[NK + NV];
    auto read = [&](int r) {
        if (r < NK) {
            rd[r] = ds_read16(koff[r % NS] + kt + (r / NS) * 8192);
        } else if (r < NK + NV) {
            const int s4 = (r - NK) / NDB, db = (r - NK) % NDB;
            rd[r] = ds_read_tr16x2(voff[db].x + vt + 4096 * s4, voff[db].y + vt + 4096 * s4);
        }
    };
#pragma unroll
    for (int r = 0; r < PF; ++r) read(r);

    f32x16 s0[2] = {f32x16{}, f32x16{}}, s1[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        s0[0] = mfma32x32x16(rd[j], qf[0][j], s0[0]);
        s0[1] = mfma32x32x16(rd[j], qf[1][j], s0[1]);
        read(j + PF);
    }
#pragma unroll
    for (int j = NS; j < NK; ++j) {
        s1[0] = mfma32x32x16(rd[j], qf[0][j - NS], s1[0]);
        s1[1] = mfma32x32x16(rd[j], qf[1][j - NS], s1[1]);
        read(j + PF);
    }
    uint4 p0[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) p0[rb][kk] = silu_operand<MASKED>(s0[rb], 8 * kk, n0, lim[rb], g);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
        const int kk = i / NDB, db = i % NDB;
        oacc[db][0] = mfma32x32x16(rd[NK + i], p0[0][kk], oacc[db][0]);
        oacc[db][1] = mfma32x32x16(rd[NK + i], p0[1][kk], oacc[db][1]);
        read(NK + i + PF);
    }
    uint4 p1[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) p1[rb][kk] = silu_operand<MASKED>(s1[rb], 8 * kk, n0 + 32, lim[rb], g);
#pragma unroll
    for (int i = 2 * NDB; i < NV; ++i) {
        const int kk = i / NDB - 2, db = i % NDB;
        oacc[db][0] = mfma32x32x16(rd[NK + i], p1[0][kk], oacc[db][0]);
        oacc[db][1] = mfma32x32x16(rd[NK + i], p1[1][kk], oacc[db][1]);
        read(NK + i + PF);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int NDB = DM / 32;
    constexpr int KSTEPS = D / 16;
    // [pair 0: K slot 0 | K slot 1 | V slot 0 | V slot 1][pair 1: same]
    __shared__ __attribute__((aligned(16))) uint16_t smem[8 * kTileElems];
    const uint32_t lds0 = lds_addr(smem);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int rg = wave & 1;   // row half of the block
    const int kg = wave >> 1;  // key tile parity, and wave pair
    const uint32_t grp = lds0 + (uint32_t)kg * kGroupBytes;

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
    const int row0 = m0 + 64 * rg;  // first row of this wave
    const bool wave_live = row0 < sb.lq;
    int lim[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) lim[rb] = CAUSAL ? min(kv_end, row0 + 32 * rb + l32 + 1) : kv_end;

    uint4 qf[2][KSTEPS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = min(row0 + 32 * rb + l32, sb.lq - 1);
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[rb][kk] = scale_bf16x8(ld_global16(src + 16 * kk), p.exp_c);
    }
    uint32_t koff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = grp + tile_byte(l32, 2 * kk + g);
    uint2 voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        voff[db] = tr_offsets(32 * db, lane);
        voff[db].x += grp + 2 * kTileBytes;
        voff[db].y += grp + 2 * kTileBytes;
    }
    f32x16 oacc[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db][0] = oacc[db][1] = f32x16{};

    if (ntiles > 0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D, 2> kdma, vdma;
        kdma.init(rg, lane, p.k.tok);
        vdma.init(rg, lane, p.v.tok);
        if constexpr (D < 32) {
            // columns D..31 of every slot are read by the 32-wide MFMA blocks
            constexpr int U = kTileRows * (32 - D) / 8;  // 16-byte units per slot
            for (int u = tid; u < 8 * U; u += 256) {
                const int sl = u / U, v = u % U;
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        if (kg < ntiles) {
            kdma.issue(grp, kbase, p.k.tok, kg * BN, kv_end);
            vdma.issue(grp + 2 * kTileBytes, vbase, p.v.tok, kg * BN, kv_end);
        }
        wait_global_loads();
        __syncthreads();

        // Every step but the last is free of masking for every wave: for a causal
        // block m the first tile that crosses a wave's diagonal is tile 2m, in the
        // last step; without a causal mask only the last tile can pass the
        // sequence end.  The last step runs the masked variant for all waves.
        const int nsteps = (ntiles + 1) / 2;
        auto step = [&](int s, auto masked) {
            const int t = 2 * s + kg;  // this pair's tile
            const uint32_t cur = (uint32_t)(s & 1) * kTileBytes, nxt = kTileBytes - cur;
            if (t + 2 < ntiles) {  // the other slots were last read before the previous barrier
                kdma.issue(grp + nxt, kbase, p.k.tok, (t + 2) * BN, kv_end);
                vdma.issue(grp + 2 * kTileBytes + nxt, vbase, p.v.tok, (t + 2) * BN, kv_end);
            }
            const int n0 = t * BN;
            // waves whose rows all precede the tile's first key, or lie past the sequence, skip it
            if (t < ntiles && wave_live && !(CAUSAL && n0 > row0 + 63))
                fwd_tile<D, decltype(masked)::value>(cur, cur, qf, oacc, koff, voff, n0, lim, g);
            wait_global_loads();
            __syncthreads();
        };
        for (int s = 0; s + 1 < nsteps; ++s) step(s, std::false_type{});
        step(nsteps - 1, std::true_type{});

        // the odd-tile pair hands its partial sums to the even-tile pair through LDS
        if (ntiles > 1) {
            const uint32_t red = lds0 + (uint32_t)rg * (NDB * 2 * 16 * 64 * 4) + 16u * lane;
            if (kg == 1) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const f32x16& a = oacc[db][rb];
                            ds_write16(red + (uint32_t)(((db * 2 + rb) * 4 + j) * 1024),
                                       make_uint4(__float_as_uint(a[4 * j]), __float_as_uint(a[4 * j + 1]),
                                                  __float_as_uint(a[4 * j + 2]), __float_as_uint(a[4 * j + 3])));
                        }
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint4 w = ds_read16(red + (uint32_t)(((db * 2 + rb) * 4 + j) * 1024));
                            oacc[db][rb][4 * j] += __uint_as_float(w.x);
                            oacc[db][rb][4 * j + 1] += __uint_as_float(w.y);
                            oacc[db][rb][4 * j + 2] += __uint_as_float(w.z);
                            oacc[db][rb][4 * j + 3] += __uint_as_float(w.w);
                        }
            }
        }
    }

    if (kg != 0) return;
    const float sc = p.pre_scale;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int my_row = row0 + 32 * rb + l32;
        if (my_row < sb.lq) {
            uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int d0 = db * 32 + 8 * rq + 4 * g;
                    if (d0 < D) {
                        const f32x16& a = oacc[db][rb];
                        const uint2 w = make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                                   pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                        *reinterpret_cast<uint2*>(dst + d0) = w;
                    }
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
