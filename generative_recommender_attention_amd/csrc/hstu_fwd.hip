// HSTU attention forward on gfx950.
//
// Computes, per packed sequence and head (HSTU Attention page, "Overview"
// equations), O = ((M (.) SiLU(alpha Q K^T)) / L_scale) V with no softmax, so no
// running maximum, no rescaling and no row statistics are kept: O is a plain
// sum over key tiles.
//
// Workgroup = 4 wavefronts, two workgroups per CU = 128 query rows of one
// (sequence, head); wave w owns rows 32 w .. 32 w + 31.  Grid = (live row block,
// head), head fastest, over the live blocks in the order of find_block: block
// index descending, so that under a causal mask the blocks with the most key
// tiles start first; the host never reads the cumulative lengths and the
// surplus workgroups sit at the end of the grid.
//
// The mask ("Mask support" table) decides the block's key range and which tiles
// need the per-element test: full attention walks every key tile and tests only
// the sequence end; causal stops at the block's diagonal and tests only its last
// two tiles; a token window (left, right) walks the tiles that meet the band of
// its rows, [first row - left, last row + right], and each wave decides per tile
// whether the band covers the tile for all its rows (no test), misses it for all
// (skip) or cuts it (test each score against the row's own interval).  The
// arbitrary interval mask walks the tiles between the smallest and the largest
// visible key of the block's rows; per tile each lane forms its row's 64-bit
// key mask from the row's endpoints, and two ballots over the wave's live rows
// choose skip, no test, or a bit test per score.
//
// K and V tiles (64 keys x D, row-major, swizzled) are staged into LDS with
// direct global->LDS loads issued from inline assembly, double-buffered: the
// loads of the next tile are issued before the current one is computed and
// waited for (vmcnt) before the one barrier per step.  Per tile a wave runs, for
// each 32-key half,
//   X^T (32 x 32)  = K_half Q^T      on MFMA: A = K rows from LDS, B = Q from
//                    registers (both exact bf16, so X = Q K^T is the fp32 sum)
//   P^T            = bf16(x / (1 + 2^(c x))), c = -alpha log2 e applied in fp32,
//                    masked on edge tiles only
//   O^T (D x 32)  += V_half^T P^T    on MFMA: A = V read transposed from LDS
// with the scores of one half turned into P^T while the next half's products
// run, and the epilogue writing O = (alpha / L_scale) O^T^T in bf16.
#include <type_traits>

#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;                   // 128 query rows per workgroup
constexpr int BN = kTileRows;                    // 64 keys per tile
constexpr uint32_t kTileBytes = 2 * kTileElems;  // 16 KB per staged 64-row tile

// How a tile's scores are masked: not at all; against this lane's key interval
// [lo, lo + span) (one unsigned compare tests both ends); or, when the wave-uniform
// flag is set, against a bit word per 32-key block (bit 8 (r / 4) + r % 4 of the
// word, pre-shifted by 4 g, is the key of accumulator register r).
enum TileMask : int { kNoMask = 0, kInterval = 1, kBits = 2 };

// bf16 P^T operand from accumulator registers r0..r0+7 of a 32-key block whose
// first key is key0.  The registers hold raw scores x = q.k; SiLU(alpha x) /
// alpha = x / (1 + 2^(c x)), c = -alpha log2(e), costs two multiplies, one exp,
// one add and one rcp; the factor alpha goes into the output scale.  Scaling the
// scores in fp32 (rather than a bf16 operand by c) keeps them exact to fp32
// rounding.  kInterval: (a, b) = (lo, span); kBits: a = the block's bit word, b the flag.
template <int MT>
__device__ __forceinline__ uint4 silu_operand(const f32x16& s, int r0, int key0, int a, int b, int g, float c) {
    float pv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pv[r] = silu_x(s[r0 + r], c);
    if constexpr (MT == kInterval) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            pv[r] = (unsigned)(key0 + acc_row(r0 + r, g) - a) < (unsigned)b ? pv[r] : 0.0f;
    } else if constexpr (MT == kBits) {
        if (b) {
            keep_branch();
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int bit = 8 * ((r0 + r) >> 2) + ((r0 + r) & 3);
                pv[r] = ((unsigned)a >> bit) & 1u ? pv[r] : 0.0f;
            }
        }
    }
    return pack_operand(pv);
}

// One 64-key tile for one wave of 32 query rows.  S^T for the first 32 keys
// (s0), then for the second 32 (s1); P^T of s0 is computed while s1's products
// run, the first half of O^T += V^T P^T while P^T of s1 is computed.  Reads are
// issued in product order, PF ahead of the MFMA that uses them.
template <int D, int MT, uint32_t kt, uint32_t vt>
__device__ __forceinline__ void fwd_tile(const uint4 (&qf)[D / 16],
                                         f32x16 (&oacc)[(D < 32 ? 32 : D) / 32], const uint32_t (&koff)[D / 16],
                                         const uint2 (&voff)[(D < 32 ? 32 : D) / 32], int n0, int a0, int b0,
                                         int a1, int b1, int g, float c) {
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
    const uint4 p0 = silu_operand<MT>(s0, 0, n0, a0, b0, g, c);
    const uint4 p1 = silu_operand<MT>(s0, 8, n0, a0, b0, g, c);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < NDB ? p0 : p1, oacc[i % NDB]);
        read(NK + i + PF);
    }
    const uint4 p2 = silu_operand<MT>(s1, 0, n0 + 32, a1, b1, g, c);
    const uint4 p3 = silu_operand<MT>(s1, 8, n0 + 32, a1, b1, g, c);
#pragma unroll
    for (int i = 2 * NDB; i < NV; ++i) {
        oacc[i % NDB] = mfma32x32x16(rd[NK + i], i < 3 * NDB ? p2 : p3, oacc[i % NDB]);
        read(NK + i + PF);
    }
}

template <int D, MaskKind MK>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnParams p) {
    constexpr bool CAUSAL = MK == MaskKind::Causal;
    constexpr bool WINDOW = MK == MaskKind::Window;
    constexpr bool FUNC = MK == MaskKind::Func;
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int NDB = DM / 32;
    constexpr int KSTEPS = D / 16;
    // [K slot 0 | K slot 1 | V slot 0 | V slot 1]
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTileElems];
    __shared__ int kv_red[FUNC ? 8 : 1];  // func: per-wave key range of the block's rows
    const uint32_t lds0 = lds_addr(smem);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const float c = p.exp_c;

    // workgroup -> (live row block, head), head fastest; surplus workgroups exit
    const int h = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.heads));
    BlockItem item;
    const int pidx = (int)(blockIdx.x / (unsigned)p.heads);
    if (!(CAUSAL || MK == MaskKind::None
              ? find_block_by_cost<true>(p.cu_q, p.cu_k, p.batch, p.max_cost, pidx, QueryBlocksGe<BM, CAUSAL>{p.max_cost}, item)
              : find_block<true>(p.cu_q, p.batch, BM, p.nblk, pidx, item)))
        return;
    const int b = item.b, m = item.m;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    dbg_seq(p, sb, h);
    const int m0 = m * BM;
    const int row0 = m0 + 32 * wave;  // first row of this wave
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;

    // Keys [kv_begin, kv_end) some row of the block sees, and this lane's own
    // interval [lo, lo + span).
    int kv_begin = 0, kv_end = sb.lk, lo = 0, span;
    // window only: keys every live row of the wave sees [full_lo, full_hi), and
    // keys some live row of the wave sees [any_lo, any_hi)
    int full_lo = 0, full_hi = 0, any_lo = 0, any_hi = 0;
    int f0 = 0, f1 = 0, f2 = 0;  // func: this lane's first endpoints, kept for the whole walk
    if constexpr (WINDOW) {
        const int L = p.win_left, R = p.win_right;
        const int last = min(m0 + BM, sb.lq) - 1;
        kv_begin = max(0, m0 - L);
        kv_end = max(kv_begin, min(sb.lk, last + R + 1));
        lo = max(0, my_row - L);
        span = max(0, min(sb.lk, my_row + R + 1) - lo);
        const int wlast = min(row0 + 31, sb.lq - 1);
        full_lo = max(0, wlast - L);
        full_hi = min(sb.lk, row0 + R + 1);
        any_lo = max(0, row0 - L);
        any_hi = min(sb.lk, wlast + R + 1);
    } else if constexpr (FUNC) {
        // keys between the smallest and the largest visible key of any row of the block
        int rlo = 0x7fffffff, rhi = 0;
        if (my_row < sb.lq) func_key_range(p.func, p.func_ld, p.func_n, sb.q0 + my_row, sb.lk, rlo, rhi);
        const int frow = sb.q0 + min(my_row, sb.lq - 1);
        HSTU_DCHECK(frow >= 0 && frow < p.func_ld, kDbgFunc);
        f0 = p.func[frow];
        if (p.func_n > 1) {
            f1 = p.func[(int64_t)p.func_ld + frow];
            f2 = p.func[2 * (int64_t)p.func_ld + frow];
        }
        rlo = wave_min(rlo);
        rhi = wave_max(rhi);
        if (lane == 0) {
            kv_red[2 * wave] = rlo;
            kv_red[2 * wave + 1] = rhi;
        }
        __syncthreads();
        kv_begin = min(min(kv_red[0], kv_red[2]), min(kv_red[4], kv_red[6]));
        kv_end = max(max(kv_red[1], kv_red[3]), max(kv_red[5], kv_red[7]));
        span = 0;
    } else {
        if (CAUSAL) kv_end = min(sb.lk, m0 + BM);
        span = CAUSAL ? min(kv_end, my_row + 1) : kv_end;
    }
    const int t0 = kv_end > kv_begin ? kv_begin / BN : 0;
    const int ntiles = kv_end > kv_begin ? (kv_end + BN - 1) / BN - t0 : 0;
    HSTU_DCHECK(ntiles == 0 || (kv_begin >= 0 && kv_end <= sb.lk), kDbgTile);

    uint4 qf[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        HSTU_DCHECK(r >= 0 && r < sb.lq, kDbgRow);
        const uint16_t* src = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = ld_global16(src + 16 * kk);
    }
    uint32_t koff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = lds0 + tile_byte(l32, 2 * kk + g);
    uint2 voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        voff[db] = tr_offsets(32 * db, lane);
        voff[db].x += lds0 + 2 * kTileBytes;
        voff[db].y += lds0 + 2 * kTileBytes;
    }
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

    if (ntiles > 0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D> kdma, vdma;
        kdma.init(wave, lane, p.k.tok);
        vdma.init(wave, lane, p.v.tok);
        if constexpr (D < 32) {
            // columns D..31 of every slot are read by the 32-wide MFMA blocks
            constexpr int U = kTileRows * (32 - D) / 8;  // 16-byte units per slot
            for (int u = tid; u < 4 * U; u += 256) {
                const int sl = u / U, v = u % U;
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        kdma.issue(lds0, kbase, p.k.tok, t0 * BN, kv_end);
        vdma.issue(lds0 + 2 * kTileBytes, vbase, p.v.tok, t0 * BN, kv_end);
        wait_global_loads();
        __syncthreads();

        // Step s computes tile t0 + s from slot s % 2 while tile t0 + s + 1 streams
        // into the other slot.  Without a window only the tiles that cross a
        // wave's diagonal or the sequence end need the per-element mask, and those
        // are the block's last two tiles: for a causal block m the first tile
        // crossing a diagonal is tile 2m of 2m + 2; without a causal mask only the
        // last tile can pass the sequence end.  Slots alternate at compile time so
        // that every LDS offset is an immediate.
        const int nplain = WINDOW || FUNC ? ntiles : ntiles - min(ntiles, 2);
        auto step = [&](int s, auto slot, auto masked) {
            constexpr uint32_t cur = decltype(slot)::value * kTileBytes, nxt = kTileBytes - cur;
            if (s + 1 < ntiles) {  // the other slots were last read before the previous barrier
                kdma.issue(lds0 + nxt, kbase, p.k.tok, (t0 + s + 1) * BN, kv_end);
                vdma.issue(lds0 + 2 * kTileBytes + nxt, vbase, p.v.tok, (t0 + s + 1) * BN, kv_end);
            }
            const int n0 = (t0 + s) * BN;
            if constexpr (WINDOW) {
                if (wave_live && n0 + BN > any_lo && n0 < any_hi) {
                    if (n0 >= full_lo && n0 + BN <= full_hi)
                        fwd_tile<D, kNoMask, cur, cur>(qf, oacc, koff, voff, n0, 0, 0, 0, 0, g, c);
                    else
                        fwd_tile<D, kInterval, cur, cur>(qf, oacc, koff, voff, n0, lo, span, lo, span, g, c);
                }
            } else if constexpr (FUNC) {
                // this lane's visible keys of the tile; the live rows of the wave decide
                // between skipping the tile, the unmasked code and the bit-masked code
                if (wave_live) {
                    const bool live = my_row < sb.lq;
                    const uint64_t bits = func_bits64_pre(f0, f1, f2, p.func, p.func_ld, p.func_n,
                                                          sb.q0 + min(my_row, sb.lq - 1), n0, sb.lk);
                    const uint64_t seen = __ballot(live && bits != 0);
                    const int cut = __ballot(live && bits != ~0ull) != 0;
                    if (seen != 0) {
                        const uint64_t sh = bits >> (4 * g);
                        fwd_tile<D, kBits, cur, cur>(qf, oacc, koff, voff, n0, (int)(uint32_t)sh, cut,
                                                     (int)(uint32_t)(sh >> 32), cut, g, c);
                    }
                }
            } else {
                // waves whose rows all precede the tile's first key, or lie past the sequence, skip it
                if (wave_live && !(CAUSAL && n0 > row0 + 31))
                    fwd_tile<D, decltype(masked)::value ? kInterval : kNoMask, cur, cur>(qf, oacc, koff, voff, n0, lo,
                                                                                         span, lo, span, g, c);
            }
            wait_global_loads();
            __syncthreads();
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        for (int s = 0; s < nplain; s += 2) {
            step(s, S0{}, std::false_type{});
            if (s + 1 < nplain) step(s + 1, S1{}, std::false_type{});
        }
        for (int s = nplain; s < ntiles; ++s) {
            if (s & 1) step(s, S1{}, std::true_type{});
            else step(s, S0{}, std::true_type{});
        }
    }

    if (my_row >= sb.lq) return;
    HSTU_DCHECK((int64_t)sb.q0 + my_row < p.total_q, kDbgRow);
    uint16_t* dst = p.o.base + (int64_t)(sb.q0 + my_row) * p.o.tok + (int64_t)h * p.o.head;
    const float sc = p.out_scale;
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

template <int D, MaskKind MK>
hipError_t launch(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.items * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_kernel<D, MK>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, MaskKind mask, hipStream_t stream) {
    switch (mask) {
        case MaskKind::None: return launch<D, MaskKind::None>(p, stream);
        case MaskKind::Causal: return launch<D, MaskKind::Causal>(p, stream);
        case MaskKind::Window: return launch<D, MaskKind::Window>(p, stream);
        case MaskKind::Func: return launch<D, MaskKind::Func>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

#ifdef HSTU_DEBUG
hipError_t debug_take_fwd(uint32_t* out) { return dbg_take(out); }
#endif

hipError_t launch_fwd(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream) {
    switch (head_dim) {
        case 16: return launch_d<16>(p, mask, stream);
        case 32: return launch_d<32>(p, mask, stream);
        case 64: return launch_d<64>(p, mask, stream);
        case 128: return launch_d<128>(p, mask, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hstu
