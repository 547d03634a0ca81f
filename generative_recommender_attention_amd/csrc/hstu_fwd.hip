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
// through LDS at the end.  Grid = (live row block, head), head fastest, over
// the live blocks in the order of find_block: block index descending, so the
// blocks with the most key tiles start first; the host never reads the
// cumulative lengths and the surplus workgroups sit at the end of the grid.
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

// One 64-key tile for one wave of 32 query rows.  S^T for the first 32 keys
// (s0), then for the second 32 (s1); P^T of s0 is computed while s1's products
// run, the first half of O^T += V^T P^T while P^T of s1 is computed.  Reads are
// issued in product order, PF ahead of the MFMA that uses them.
template <int D, bool MASKED, uint32_t kt, uint32_t vt>
__device__ __forceinline__ void fwd_tile(const uint4 (&qf)[D / 16],
                                         f32x16 (&oacc)[(D < 32 ? 32 : D) / 32], const uint32_t (&koff)[D / 16],
                                         const uint2 (&voff)[(D < 32 ? 32 : D) / 32], int n0, int lim, int g) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;  // 32-column blocks of O^T
    constexpr int NS = D / 16;                   // contraction steps per S^T block
    constexpr int NK = 2 * NS;                   // K reads: block-major, step-minor
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
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        if (j < NS) s0 = mfma32x32x16(rd[j], qf[j], s0);
        else s1 = mfma32x32x16(rd[j], qf[j - NS], s1);
        read(j + PF);
    }
    const uint4 p0 = silu_operand<MASKED>(s0, 0, n0, lim, g);
    const uint4 p1 = silu_operand<MASKED>(s0, 8, n0, lim, g);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < NDB ? p0 : p1, oacc[i % NDB]);
        read(NK + i + PF);
    }
    const uint4 p2 = silu_operand<MASKED>(s1, 0, n0 + 32, lim, g);
    const uint4 p3 = silu_operand<MASKED>(s1, 8, n0 + 32, lim, g);
#pragma unroll
    for (int i = 2 * NDB; i < NV; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < 3 * NDB ? p2 : p3, oacc[i % NDB]);
        read(NK + i + PF);
    }
}

template <int D, bool CAUSAL, int KSPLIT>
__global__ __launch_bounds__(256 * KSPLIT, 2 / KSPLIT) void fwd_kernel(AttnParams p) {
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int NDB = DM / 32;
    constexpr int KSTEPS = D / 16;
    // [group 0: K slot 0 | K slot 1 | V slot 0 | V slot 1][group 1: same]
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * KSPLIT * kTileElems];
    const uint32_t lds0 = lds_addr(smem);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const int rb = wave & 3;   // 32-row block of the workgroup's rows
    const int kg = KSPLIT == 1 ? 0 : wave >> 2;  // key tile parity, and wave group
    const uint32_t grp = lds0 + (uint32_t)kg * kGroupBytes;

    // workgroup -> (live row block, head), head fastest; surplus workgroups exit
    const int h = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.heads));
    BlockItem item;
    if (!find_block<true>(p.cu_q, p.batch, BM, p.nblk, (int)(blockIdx.x / (unsigned)p.heads), item)) return;
    const int b = item.b, m = item.m;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    const int m0 = m * BM;

    const int kv_end = CAUSAL ? min(sb.lk, m0 + BM) : sb.lk;
    const int ntiles = (kv_end + BN - 1) / BN;
    const int row0 = m0 + 32 * rb;  // first row of this wave
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;
    const int lim = CAUSAL ? min(kv_end, my_row + 1) : kv_end;

    uint4 qf[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = scale_bf16x8(ld_global16(src + 16 * kk), p.exp_c);
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
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

    if (ntiles > 0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D> kdma, vdma;
        kdma.init(rb, lane, p.k.tok);
        vdma.init(rb, lane, p.v.tok);
        if constexpr (D < 32) {
            // columns D..31 of every slot are read by the 32-wide MFMA blocks
            constexpr int U = kTileRows * (32 - D) / 8;  // 16-byte units per slot
            for (int u = tid; u < 4 * KSPLIT * U; u += 256 * KSPLIT) {
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

        // Step s: group kg computes tile t = KSPLIT s + kg from slot s % 2 while the
        // tile after it (t + KSPLIT) streams into the other slot.  Only the tiles
        // that cross a wave's diagonal or the sequence end need the per-element
        // mask, and those are the block's last two tiles: for a causal block m the
        // first tile crossing a diagonal is tile 2m of 2m + 2; without a causal
        // mask only the last tile can pass the sequence end.  They fall in the
        // last step when two groups split the tiles, in the last two otherwise.
        // Slots alternate at compile time so that every LDS offset is an immediate.
        const int nsteps = (ntiles + KSPLIT - 1) / KSPLIT;
        const int nplain = nsteps - min(nsteps, KSPLIT == 1 ? 2 : 1);
        auto step = [&](int s, auto slot, auto masked) {
            constexpr uint32_t cur = decltype(slot)::value * kTileBytes, nxt = kTileBytes - cur;
            const int t = KSPLIT * s + kg;  // this group's tile
            if (t + KSPLIT < ntiles) {  // the other slots were last read before the previous barrier
                kdma.issue(grp + nxt, kbase, p.k.tok, (t + KSPLIT) * BN, kv_end);
                vdma.issue(grp + 2 * kTileBytes + nxt, vbase, p.v.tok, (t + KSPLIT) * BN, kv_end);
            }
            const int n0 = t * BN;
            // waves whose rows all precede the tile's first key, or lie past the sequence, skip it
            if (t < ntiles && wave_live && !(CAUSAL && n0 > row0 + 31))
                fwd_tile<D, decltype(masked)::value, cur, cur>(qf, oacc, koff, voff, n0, lim, g);
            wait_global_loads();
            __syncthreads();
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        for (int s = 0; s < nplain; s += 2) {
            step(s, S0{}, std::false_type{});
            if (s + 1 < nplain) step(s + 1, S1{}, std::false_type{});
        }
        for (int s = nplain; s < nsteps; ++s) {
            if (s & 1) step(s, S1{}, std::true_type{});
            else step(s, S0{}, std::true_type{});
        }

        // the odd-tile group hands its partial sums to the even-tile group through LDS
        if (KSPLIT > 1 && ntiles > 1) {
            const uint32_t red = lds0 + (uint32_t)rb * (NDB * 16 * 64 * 4) + 16u * lane;
            if (kg == 1) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f32x16& a = oacc[db];
                        ds_write16(red + (uint32_t)((db * 4 + j) * 1024),
                                   make_uint4(__float_as_uint(a[4 * j]), __float_as_uint(a[4 * j + 1]),
                                              __float_as_uint(a[4 * j + 2]), __float_as_uint(a[4 * j + 3])));
                    }
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 w = ds_read16(red + (uint32_t)((db * 4 + j) * 1024));
                        oacc[db][4 * j] += __uint_as_float(w.x);
                        oacc[db][4 * j + 1] += __uint_as_float(w.y);
                        oacc[db][4 * j + 2] += __uint_as_float(w.z);
                        oacc[db][4 * j + 3] += __uint_as_float(w.w);
                    }
            }
        }
    }

    if (kg != 0 || my_row >= sb.lq) return;
    uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
    const float sc = p.pre_scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d0 = db * 32 + 8 * rq + 4 * g;
            if (d0 < D) {
                const f32x16& a = oacc[db];
                const uint2 w = make_uint2(pack_bf16x2(a[4 * rq] * sc, a[4 * rq + 1] * sc),
                                           pack_bf16x2(a[4 * rq + 2] * sc, a[4 * rq + 3] * sc));
                *reinterpret_cast<uint2*>(dst + d0) = w;
            }
        }
    }
}

#ifndef HSTU_FWD_KSPLIT
#define HSTU_FWD_KSPLIT 1
#endif
template <int D, bool CAUSAL>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
    constexpr int KSPLIT = HSTU_FWD_KSPLIT;
    const int64_t grid = (int64_t)p.nblk * p.batch * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, KSPLIT>), dim3((unsigned)grid), dim3(256 * KSPLIT), 0, stream, p);
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
