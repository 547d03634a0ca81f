// HSTU attention backward on gfx950.  Three routes: a dq kernel and a dk/dv kernel
// that both recompute the scores (no workspace); given a workspace, the dk/dv
// kernel storing dS and a dq kernel that reads it (described last) -- both of
// these deterministic, with no atomics; and the fused backward, one dk/dv pass
// that also adds each query tile's dQ into an fp32 accumulator with atomics (the
// HSTU page's form for D <= 128, whose dQ summation order is not fixed).
//
// The backward receives dO and q, k, v only (HSTU Attention page, "High-level
// functions"), so both kernels recompute the scores.  With s = alpha q_i.k_j,
// a = SiLU(s) / L_scale and dA_ij = dO_i . v_j (chain rule on the page's
// "Overview" equations):
//     dV_j = sum_i M_ij a_ij dO_i
//     dQ_i = alpha sum_j M_ij dA_ij SiLU'(s_ij) / L_scale k_j
//     dK_j = alpha sum_i M_ij dA_ij SiLU'(s_ij) / L_scale q_i
// SiLU'(s) = sig(s) (1 + s (1 - sig(s))).  As in the forward, the score MFMAs
// run on the exact bf16 q and k, so they produce x = q_i.k_j to fp32 rounding,
// and alpha is applied in fp32: sig(s) = 1 / (1 + 2^(c x)) with c = -alpha log2 e;
// alpha / L_scale is applied at the final stores of dQ, dK and dV.
//
// dq kernel: query-major, one workgroup per (128-row block, sequence, head), the
// same tile walk and mask handling as the forward, two workgroups per CU (so the
// exponent work of one overlaps the products of the other).  Per 64-key tile K and V are staged
// row-major in LDS; each wave computes S^T = K Q^T and dA^T = V dO^T (A operands:
// K, V rows), forms dS^T in registers and accumulates dQ^T += K^T dS^T (A
// operand: K read transposed).
//
// dk/dv kernel: key-major, one 8-wave workgroup per (128-key block, sequence,
// head).  The block's K and V rows sit in LDS for the whole walk;
// waves w and w + 4 own the same 32 keys and take the first and second 32 rows
// of every query tile, so each wave holds only its dK^T and dV^T accumulators
// and two waves fit per SIMD; their partial sums are added through LDS at the
// end.  Causal blocks walk query tiles from the block's first key to the end of
// the sequence (rows before it see none of these keys); under a token window
// (left, right) they walk rows [first key - right, last key + left], the rows
// whose band meets the block (the start rounded down to a multiple of 32, so
// that row blocks line up with the stored dS blocks), and each wave tests per
// 32-row block whether the band covers, misses or cuts it, as the forward does.  Under the arbitrary
// interval mask they walk the rows between the first and the last row of the
// sequence that sees a key of the block (a scan of its rows' endpoints), and
// 256 threads turn each query tile's endpoints into 64 x 4 visibility words in
// LDS (32 keys each, double-buffered beside the tile) that each wave reads to
// classify its 32-row block and, when cut, to test each score.  Per 64-row query tile
// Q and dO are staged row-major; each wave computes S = Q K^T and dA = dO V^T
// (A operands: Q, dO rows; B operands: K, V rows), forms A' and dS in registers
// and accumulates dV^T += dO^T A' and dK^T += Q^T dS (A operands: dO, Q read
// transposed).
//
// Tiles are staged as in the forward: one LDS array with two slots per operand,
// direct global->LDS loads issued from inline assembly (tile t+1 loads while
// tile t is computed) and byte-addressed reads issued a few products ahead of
// their MFMAs.  Splitting the gradients over two kernels executes 14 D flops
// per visible pair against 10 D for a single pass, but needs no atomics and no
// workspace and is bit-for-bit reproducible.
//
// Stored dS: the dk/dv kernel also writes each 32 x 32 block of bf16 dS it forms
// (the dS^T operand of its dK product, as it sits in the registers: 2 bytes per
// visible pair, streamed past the caches), and the second dq kernel computes
// dQ^T = K^T dS^T from those blocks: 2 D flops per pair instead of 6 D, no
// exponentials, and no Q, dO or V reads, for 4 bytes of HBM traffic per pair
// (written once, read once).  The blocks keep the dk/dv kernel's orientation
// (a row per key); the dq kernel stages them in LDS and transposes them with the
// same transposing read it uses for K.  dK and dV are those of the recompute
// route bit for bit; dQ differs only in rounding (its dS comes from the scores
// as the dk/dv kernel forms them).
#include <algorithm>

#include "hstu_kernels.h"

namespace hstu {
namespace {

constexpr int BM = kFwdBlockM;   // dq kernel: query rows per workgroup (32 per wave)
constexpr int BN = kTileRows;    // dq kernel: keys per tile
constexpr int BNK = kBwdBlockN;  // dk/dv kernel: keys per workgroup (32 per wave pair)
constexpr int BMQ = kTileRows;   // dk/dv kernel: query rows per tile

// SiLU'(s) = sig (1 + s (1 - sig)) at s = alpha x, from a = x sig: s sig = alpha a,
// so SiLU'(s) = sig + alpha (a - a sig), two fused multiply-adds.
__device__ __forceinline__ float dsilu_from(float a, float sig, float alpha) {
    return __builtin_fmaf(alpha, __builtin_fmaf(-a, sig, a), sig);
}

constexpr uint32_t kTileBytes = 2 * kTileElems;  // 16 KB per staged 64-row tile

// How the dq kernel masks a 32-key block: kNoMask never; kInterval (full or
// causal) when the block reaches past wlim, the end of the keys every row of the
// wave sees, against this lane's keys [0, span); kBand (token window) when the
// block leaves [wlo, wlim), against [lo, lo + span); kBits when the wave-uniform
// flag `span` is set, against the block's bit word `lo` (pre-shifted by 4 g: bit
// 8 (r / 4) + r % 4 is the key of accumulator register r).
enum DqMask : int { kNoMask = 0, kInterval = 1, kBand = 2, kBits = 3 };

// dS^T operands of one 32-key block from its score and dA accumulators, masked
// as MT says.
template <int MT>
__device__ __forceinline__ void dq_ds_op(const f32x16& sacc, const f32x16& dacc, int key0, int lo, int span, int wlo,
                                         int wlim, int g, float c, float alpha, uint4& d0, uint4& d1) {
    float dv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float sg = sig_x(sacc[r], c);
        dv[r] = dacc[r] * dsilu_from(sacc[r] * sg, sg, alpha);
    }
    if constexpr (MT == kBits) {
        if (span) {
            keep_branch();
#pragma unroll
            for (int r = 0; r < 16; ++r) dv[r] = ((unsigned)lo >> (8 * (r >> 2) + (r & 3))) & 1u ? dv[r] : 0.0f;
        }
    } else if constexpr (MT != kNoMask) {
        if ((MT == kBand && key0 < wlo) || key0 + 32 > wlim) {
            keep_branch();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + acc_row(r, g);
                dv[r] = (MT == kBand ? (unsigned)(key - lo) < (unsigned)span : key < span) ? dv[r] : 0.0f;
            }
        }
    }
    d0 = pack_operand(dv);
    d1 = pack_operand(dv + 8);
}

// One key tile of the dq kernel for one wave, on byte-addressed LDS slots `kt`
// (K) and `vt` (V).  Products run S^T and dA^T of both 32-key blocks, then dQ^T
// of the first block (while dS^T of the second is formed), then of the second;
// every LDS read is issued PF products ahead of its MFMA.
template <int D, int MT>
__device__ __forceinline__ void dq_tile(uint32_t kt, uint32_t vt, const uint4 (&qf)[D / 16],
                                           const uint4 (&dof)[D / 16], f32x16 (&acc)[(D < 32 ? 32 : D) / 32],
                                           const uint32_t (&koff)[D / 16], const uint2 (&toff)[(D < 32 ? 32 : D) / 32],
                                           int n0, int lo, int span, int wlo, int wlim, int lo1, int g, float c,
                                           float alpha) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;
    constexpr int NS = D / 16;
    constexpr int NA = 4 * NS;   // S and dA products: block kb, step kk, operand (K, V)
    constexpr int NQ = 4 * NDB;  // dQ products: block kb = i / (2 NDB), step s = i / NDB, column block i % NDB
    constexpr int PF = 4;
    uint4 rd[NA + NQ];
    auto read = [&](int r) {
        if (r < NA) {
            const int kb = r / (2 * NS), kk = (r / 2) % NS;
            rd[r] = ds_read16(koff[kk] + ((r & 1) ? vt : kt) + kb * 8192);
        } else if (r < NA + NQ) {
            const int i = r - NA, s4 = i / NDB, db = i % NDB;
            rd[r] = ds_read_tr16x2(toff[db].x + kt + 4096 * s4, toff[db].y + kt + 4096 * s4);
        }
    };
#pragma unroll
    for (int r = 0; r < PF; ++r) read(r);
    f32x16 sa[2], da[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        sa[kb] = f32x16{};
        da[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NS; ++kk) {
            const int r = kb * 2 * NS + 2 * kk;
            sa[kb] = mfma32x32x16(rd[r], qf[kk], sa[kb]);
            read(r + PF);
            da[kb] = mfma32x32x16(rd[r + 1], dof[kk], da[kb]);
            read(r + 1 + PF);
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        uint4 d0, d1;
        dq_ds_op<MT>(sa[kb], da[kb], n0 + 32 * kb, kb ? lo1 : lo, span, wlo, wlim, g, c, alpha, d0, d1);
#pragma unroll
        for (int j = 0; j < 2 * NDB; ++j) {
            const int i = kb * 2 * NDB + j;
            acc[i % NDB] = mfma32x32x16(rd[NA + i], j < NDB ? d0 : d1, acc[i % NDB]);
            read(NA + i + PF);
        }
    }
}

template <int D, MaskKind MK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(AttnParams p) {
    constexpr bool CAUSAL = MK == MaskKind::Causal;
    constexpr bool WINDOW = MK == MaskKind::Window;
    constexpr bool FUNC = MK == MaskKind::Func;
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int KSTEPS = D / 16;
    // [K slot 0 | K slot 1 | V slot 0 | V slot 1]; tile t lives in slot (t - t0) % 2
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kTileElems];
    __shared__ int kv_red[FUNC ? 8 : 1];  // func: per-wave key range of the block's rows
    const uint32_t lds0 = lds_addr(smem);
    constexpr uint32_t K0 = 0, K1 = kTileBytes, V0 = 2 * kTileBytes, V1 = 3 * kTileBytes;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    // workgroup -> (live row block, head), head fastest, blocks with the most key tiles first
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
    if (m0 >= sb.lq) return;

    const int row0 = m0 + 32 * wave;
    const int my_row = row0 + l32;
    const bool wave_live = row0 < sb.lq;
    // Keys [kv_begin, kv_end) some row of the block sees; this lane's interval
    // [lo, lo + span); keys every live row of the wave sees [wlo, wlim); keys
    // some live row of the wave sees [any_lo, any_hi) (window only).
    int kv_begin = 0, kv_end = sb.lk, lo = 0, span, wlo = 0, wlim, any_lo = 0, any_hi = 0;
    int f0 = 0, f1 = 0, f2 = 0;  // func: this lane's first endpoints, kept for the whole walk
    if constexpr (WINDOW) {
        const int L = p.win_left, R = p.win_right;
        const int last = min(m0 + BM, sb.lq) - 1, wlast = min(row0 + 31, sb.lq - 1);
        kv_begin = max(0, m0 - L);
        kv_end = max(kv_begin, min(sb.lk, last + R + 1));
        lo = max(0, my_row - L);
        span = max(0, min(sb.lk, my_row + R + 1) - lo);
        wlo = max(0, wlast - L);
        wlim = min(sb.lk, row0 + R + 1);
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
        wlim = 0;
    } else {
        if (CAUSAL) kv_end = min(sb.lk, m0 + BM);
        span = CAUSAL ? min(kv_end, my_row + 1) : kv_end;
        wlim = CAUSAL ? min(kv_end, row0 + 1) : kv_end;
    }
    const int t0 = kv_end > kv_begin ? kv_begin / BN : 0;
    const int t1 = kv_end > kv_begin ? (kv_end + BN - 1) / BN : t0;
    HSTU_DCHECK(t1 == t0 || (kv_begin >= 0 && kv_end <= sb.lk), kDbgTile);

    uint4 qf[KSTEPS], dof[KSTEPS];
    {
        const int r = min(my_row, sb.lq - 1);
        HSTU_DCHECK(r >= 0 && r < sb.lq, kDbgRow);
        const uint16_t* qsrc = p.q.base + (int64_t)(sb.q0 + r) * p.q.tok + (int64_t)h * p.q.head + 8 * g;
        const uint16_t* dsrc = p.dout.base + (int64_t)(sb.q0 + r) * p.dout.tok + (int64_t)h * p.dout.head + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            qf[kk] = ld_global16(qsrc + 16 * kk);
            dof[kk] = ld_global16(dsrc + 16 * kk);
        }
    }
    uint32_t koff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = lds0 + tile_byte(l32, 2 * kk + g);
    uint2 toff[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        toff[db] = tr_offsets(32 * db, lane);
        toff[db].x += lds0;
        toff[db].y += lds0;
    }
    f32x16 acc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) acc[db] = f32x16{};

    if (t1 > t0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        const uint16_t* vbase = p.v.base + (int64_t)sb.k0 * p.v.tok + (int64_t)h * p.v.head;
        TileDma<D> kdma, vdma;
        kdma.init(wave, lane, p.k.tok);
        vdma.init(wave, lane, p.v.tok);
        if constexpr (D < 32) {
            // columns D..31 of the K slots are read by the 32-wide transposed blocks
            for (int u = tid; u < 2 * kTileRows * (32 - D) / 8; u += 256) {
                const int sl = u / (kTileRows * (32 - D) / 8), v = u % (kTileRows * (32 - D) / 8);
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        kdma.issue(lds0 + K0, kbase, p.k.tok, t0 * BN, kv_end);
        vdma.issue(lds0 + V0, vbase, p.v.tok, t0 * BN, kv_end);
        wait_global_loads();
        __syncthreads();

        auto step = [&](uint32_t kc, uint32_t vc, uint32_t kn, uint32_t vn, int t) {
            const int n0 = t * BN;
            if (t + 1 < t1) {
                kdma.issue(lds0 + kn, kbase, p.k.tok, n0 + BN, kv_end);
                vdma.issue(lds0 + vn, vbase, p.v.tok, n0 + BN, kv_end);
            }
            if constexpr (FUNC) {
                // this lane's visible keys of the tile; the live rows of the wave decide
                // between skipping the tile, the unmasked code and the bit-masked code
                if (wave_live) {
                    const bool live = my_row < sb.lq;
                    const uint64_t bits = func_bits64_pre(f0, f1, f2, p.func, p.func_ld, p.func_n,
                                                          sb.q0 + min(my_row, sb.lq - 1), n0, sb.lk);
                    const uint64_t seen = __ballot(live && bits != 0);
                    const int cut = __ballot(live && bits != ~0ull) != 0;
                    const uint64_t sh = bits >> (4 * g);
                    if (seen != 0)
                        dq_tile<D, kBits>(kc, vc, qf, dof, acc, koff, toff, n0, (int)(uint32_t)sh, cut, 0, 0,
                                          (int)(uint32_t)(sh >> 32), g, p.exp_c, p.alpha);
                }
            } else {
                // waves that see no key of the tile skip it
                const bool run = WINDOW ? n0 + BN > any_lo && n0 < any_hi : !(CAUSAL && n0 > row0 + 31);
                if (wave_live && run)
                    dq_tile<D, WINDOW ? kBand : kInterval>(kc, vc, qf, dof, acc, koff, toff, n0, lo, span, wlo, wlim,
                                                           lo, g, p.exp_c, p.alpha);
            }
            wait_global_loads();
            __syncthreads();
        };
        for (int t = t0; t < t1; t += 2) {
            step(K0, V0, K1, V1, t);
            if (t + 1 < t1) step(K1, V1, K0, V0, t + 1);
        }
    }

    if (my_row < sb.lq) {
        HSTU_DCHECK((int64_t)sb.q0 + my_row < p.total_q, kDbgRow);
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

// Where a wave of the dk/dv kernel stores the dS of its 32 x 32 block: `p` is the
// block (wave-uniform; lane (l32, g) writes the 64-byte row of its key l32 from
// element 8 g); `kdead` (read when the wave-uniform `kcut` is set) whether the
// lane's key lies past the sequence (stored as 0); nothing is stored unless the
// wave-uniform `on` is set.
struct DsOut {
    uint16_t* p;
    bool on, kcut, kdead;
    uint32_t lds;  // fused backward: the block's LDS byte address instead of p
};

// Query row held at position c (0..31) of a stored dS key row, and the reverse:
// the dk/dv lane (key, g) stores its operand half h (rows 16 h + 8 (t / 4) +
// 4 g + t % 4, t = 0..7) at positions 16 h + 8 g + t, i.e. bits 2 and 3 trade places.
__device__ __forceinline__ int ds_pos_row(int c) { return (c & 0x13) | ((c & 4) << 1) | ((c & 8) >> 1); }

// Byte offsets of the transposing reads of lane `lane` in a stored block: keys
// 4 g .. 4 g + 3 (.x) and 8 + 4 g .. (.y) at position l32, i.e. the dS^T operand
// half 0 of query row ds_pos_row(l32); half 1 is 16 keys (1 KB) further.
__device__ __forceinline__ uint2 ds_tr_offsets(int lane) {
    const int grp = lane >> 4, j = lane & 15;
    const int r = 4 * (grp >> 1) + (j >> 2);
    const int c = 16 * (grp & 1) + 4 * (j & 3);
    return make_uint2((uint32_t)(r * 64 + 2 * c), (uint32_t)((r + 8) * 64 + 2 * c));
}


// One 32-row block for one wave: S = Q K^T and dA = dO V^T (A operands: Q, dO
// rows of the block; B operands: the wave's K, V rows), then dV^T += dO^T A' and
// dK^T += Q^T dS over the block's two contraction steps.  When `mask` (wave-
// uniform): MT = kInterval zeroes the rows outside this lane's [lo, hi); kBits
// tests row 8 k + 4 g + j of the block (accumulator register 4 k + j) against
// bit l32 of the LDS word at mw + 32 k + 4 j.  The bf16 dS goes to `ds` as it is
// formed (the operand of dK^T itself is left as computed).
template <int D, int MT, bool TO_LDS = false, int PF = 6>
__device__ __forceinline__ void dkdv_block(bool mask, uint32_t qrow, uint32_t drow, uint32_t krow, uint32_t vrow, uint32_t qtr,
                                            uint32_t dtr, f32x16 (&dvacc)[(D < 32 ? 32 : D) / 32],
                                            f32x16 (&dkacc)[(D < 32 ? 32 : D) / 32], const uint32_t (&roff)[D / 16],
                                            const uint2 (&toff)[(D < 32 ? 32 : D) / 32], int row0, int lo, int hi,
                                            int g, uint32_t mw, const DsOut& ds, float c, float alpha) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;
    constexpr int NS = D / 16;
    constexpr int NA = 4 * NS;   // reads for S and dA: step kk, (Q, K, dO, V)
    constexpr int NG = 4 * NDB;  // reads for dV, dK: half, column block, (dO^T, Q^T)
    // PF: LDS reads issued ahead of their products

    uint4 rd[NA + NG];
    auto read = [&](int r) {
        if (r < NA) {
            const int kk = r / 4, w = r % 4;
            const uint32_t base = w == 0 ? qrow : w == 1 ? krow : w == 2 ? drow : vrow;
            rd[r] = ds_read16(roff[kk] + base);
        } else if (r < NA + NG) {
            const int i = r - NA, half = i / (2 * NDB), db = (i / 2) % NDB;
            const uint32_t base = ((i & 1) ? qtr : dtr) + 4096 * half;
            rd[r] = ds_read_tr16x2(toff[db].x + base, toff[db].y + base);
        }
    };
#pragma unroll
    for (int r = 0; r < PF; ++r) read(r);
    f32x16 sa = f32x16{}, da = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NS; ++kk) {
        sa = mfma32x32x16(rd[4 * kk], rd[4 * kk + 1], sa);
        read(4 * kk + PF);
        read(4 * kk + 1 + PF);
        da = mfma32x32x16(rd[4 * kk + 2], rd[4 * kk + 3], da);
        read(4 * kk + 2 + PF);
        read(4 * kk + 3 + PF);
    }
    float av[16], dv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float x = sa[r], sg = sig_x(x, c);
        av[r] = x * sg;
        dv[r] = da[r] * dsilu_from(av[r], sg, alpha);
    }
    if constexpr (MT == kBits) {
        if (mask) {
            keep_branch();
            const int l32 = threadIdx.x & 31;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 w = ds_read16(mw + 32 * k);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = (ws[j] >> l32) & 1u;
                    av[4 * k + j] = ok ? av[4 * k + j] : 0.0f;
                    dv[4 * k + j] = ok ? dv[4 * k + j] : 0.0f;
                }
            }
        }
    } else if constexpr (MT == kInterval) {
        if (mask) {
            keep_branch();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + acc_row(r, g);
                const bool ok = row >= lo && row < hi;
                av[r] = ok ? av[r] : 0.0f;
                dv[r] = ok ? dv[r] : 0.0f;
            }
        }
    }
    const uint4 a[2] = {pack_operand(av), pack_operand(av + 8)};
    const uint4 d[2] = {pack_operand(dv), pack_operand(dv + 8)};
    if (ds.on) {
        // the two dS^T operand halves as they are (rows past the sequence hold 0, masked
        // above; keys past it are stored as 0), with streaming stores: dS is read once,
        // by the dq kernel, and must not push the Q and dO rows that the other key
        // blocks re-read out of the caches
        const int l = threadIdx.x & 63;
        if constexpr (TO_LDS) {
            // the fused backward keeps the block in LDS for the tile's dQ products
            const uint32_t dst = ds.lds + 64u * (uint32_t)(l & 31) + 16u * (uint32_t)(l >> 5);
            const bool dead = ds.kcut && ds.kdead;
            ds_write16(dst, dead ? make_uint4(0, 0, 0, 0) : d[0]);
            ds_write16(dst + 32u, dead ? make_uint4(0, 0, 0, 0) : d[1]);
        } else {
            uint16_t* dst = ds.p + (l & 31) * kDsRowElems + 8 * (l >> 5);
            if (ds.kcut && ds.kdead) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                __builtin_nontemporal_store(z, (global_u32x4*)dst);
                __builtin_nontemporal_store(z, (global_u32x4*)(dst + 16));
            } else {
                const u32x4 v0 = {d[0].x, d[0].y, d[0].z, d[0].w}, v1 = {d[1].x, d[1].y, d[1].z, d[1].w};
                __builtin_nontemporal_store(v0, (global_u32x4*)dst);
                __builtin_nontemporal_store(v1, (global_u32x4*)(dst + 16));
            }
        }
        // keep the stores ahead of the dV / dK products, so that they drain while
        // those run instead of in front of the tile's closing wait
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int half = j / (2 * NDB), db = (j / 2) % NDB;
        if (j & 1) dkacc[db] = mfma32x32x16(rd[NA + j], d[half], dkacc[db]);
        else dvacc[db] = mfma32x32x16(rd[NA + j], a[half], dvacc[db]);
        read(NA + j + PF);
    }
}

// Modes of the dk/dv kernel: recompute only; also store dS for the dq-from-dS
// kernel; or the fused backward, which also adds each query tile's dQ into an fp32
// accumulator with atomics (no dq kernel; dQ's summation order is not fixed).
enum DkdvMode : int { kDkdvPlain = 0, kDkdvStoreDs = 1, kDkdvFusedDq = 2 };

template <int D, MaskKind MK, int MODE>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(AttnParams p) {
    constexpr bool DS = MODE == kDkdvStoreDs;
    constexpr bool FQ = MODE == kDkdvFusedDq;
    constexpr bool CAUSAL = MK == MaskKind::Causal;
    constexpr bool WINDOW = MK == MaskKind::Window;
    constexpr bool FUNC = MK == MaskKind::Func;
    // DS: the launch stores dS (p.ds is the workspace); the row blocks of the walk then
    // start on multiples of 32 under every mask
    constexpr int DM = D < 32 ? 32 : D;
    constexpr int KSTEPS = D / 16;
    // [Q slot 0 | Q slot 1 | dO slot 0 | dO slot 1 | K rows of the block | V rows of the block]
    __shared__ __attribute__((aligned(16))) uint16_t smem[8 * kTileElems];
    // func: visibility words of a query tile, two slots of [32-key word w][64 rows]
    // (bit k of word w, row r: key n0 + 32 w + k visible to row r of the tile)
    __shared__ __attribute__((aligned(16))) uint32_t fmask[FUNC ? 2 * 256 : 4];
    __shared__ int q_red[FUNC ? 16 : 1];
    // fused backward: the tile's eight 32 x 32 dS blocks ([row half][key sub-block], in
    // the stored-dS block layout) and whether each was computed this step
    __shared__ __attribute__((aligned(16))) uint16_t fq_ds[FQ ? 8 * kDsBlockElems : 8];
    __shared__ int fq_on[FQ ? 8 : 1];
    const uint32_t lds0 = lds_addr(smem);
    constexpr uint32_t Q0 = 0, Q1 = kTileBytes, D0 = 2 * kTileBytes, D1 = 3 * kTileBytes;
    constexpr uint32_t KB = 4 * kTileBytes, VB = 6 * kTileBytes;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kw = wave & 3, qh = wave >> 2;  // key sub-block, row half of each tile
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;

    // workgroup -> (live key block, head), head fastest, blocks with the most query tiles first
    const int h = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.heads));
    BlockItem item;
    const int pidx = (int)(blockIdx.x / (unsigned)p.heads);
    if (!(CAUSAL || MK == MaskKind::None
              ? find_block_by_cost<false>(p.cu_q, p.cu_k, p.batch, p.max_cost, pidx, KeyBlocksGe<BNK, CAUSAL>{p.max_cost}, item)
              : find_block<false>(p.cu_k, p.batch, BNK, p.nblk, pidx, item)))
        return;
    const int b = item.b, n = item.m;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    dbg_seq(p, sb, h);
    const int n0 = n * BNK;
    if (n0 >= sb.lk) return;

    const int key0 = n0 + 32 * kw;
    const int my_key = key0 + l32;
    const bool wave_live = key0 < sb.lk;
    // stored dS: the sequence's first block (wave-uniform); a tile adds its block's
    // index within the sequence's share
    uint16_t* ds_base = nullptr;
    const int ds_ng = (sb.lk + 31) >> 5;  // key groups of the sequence
    if constexpr (DS) {
        const int64_t seq0 = p.ds_rel >= 0 ? (((int64_t)sb.q0 + 31 * (int64_t)b) >> 5) * p.ds_kg
                                           : ds_seq_base(p.cu_q, p.cu_k, b, p.ds_tri != 0);
        ds_base = static_cast<uint16_t*>(
            const_cast<void*>(uniform_ptr(p.ds + ((int64_t)h * p.ds_head + seq0) * kDsBlockElems)));
    }

    // the block's K and V rows into LDS; rows past the sequence repeat its last row
    for (int u = tid; u < BNK * 16; u += 512) {
        const int r = u >> 4, c = u & 15;
        if (c < D / 8) {
            const int64_t row = sb.k0 + min(n0 + r, sb.lk - 1);
            HSTU_DCHECK(row >= sb.k0 && row < (int64_t)sb.k0 + sb.lk, kDbgRow);
            const uint4 kv = ld_global16(p.k.base + row * p.k.tok + (int64_t)h * p.k.head + 8 * c);
            const uint4 vv = ld_global16(p.v.base + row * p.v.tok + (int64_t)h * p.v.head + 8 * c);
            ds_write16(lds0 + KB + tile_byte(r, c), kv);
            ds_write16(lds0 + VB + tile_byte(r, c), vv);
        }
    }
    uint32_t roff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) roff[kk] = lds0 + tile_byte(l32, 2 * kk + g);
    uint2 toff[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        toff[db] = tr_offsets(32 * db, lane);
        toff[db].x += lds0;
        toff[db].y += lds0;
    }
    f32x16 dvacc[DM / 32], dkacc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) dvacc[db] = dkacc[db] = f32x16{};

    // Query rows [q_begin, q_end) that see some key of the block; this lane's
    // rows [lo, hi); rows that see every live key of the wave [wlo, whi); rows
    // that see some live key of the wave [any_lo, any_hi) (window only).
    int q_begin = 0, q_end = sb.lq, lo = 0, hi = sb.lq, wlo = 0, whi = sb.lq, any_lo = 0, any_hi = 0;
    if constexpr (WINDOW) {
        const int L = p.win_left, R = p.win_right;
        const int last = min(n0 + BNK, sb.lk) - 1, wlast = min(key0 + 31, sb.lk - 1);
        q_begin = max(0, n0 - R) & ~31;  // 32-row aligned (rows before n0 - R see none of these keys)
        q_end = max(q_begin, min(sb.lq, last + L + 1));
        lo = max(0, my_key - R);
        hi = min(sb.lq, my_key + L + 1);
        wlo = max(0, wlast - R);
        whi = min(sb.lq, key0 + L + 1);
        any_lo = max(0, key0 - R);
        any_hi = min(sb.lq, wlast + L + 1);
    } else if constexpr (CAUSAL) {
        q_begin = n0;
        lo = my_key;
        wlo = key0 + 31;  // largest lo in the wave
    } else if constexpr (FUNC) {
        // the first and last rows of the sequence that see a key of the block
        const int k1 = min(n0 + BNK, sb.lk);
        int qlo = 0x7fffffff, qhi = -1;
        for (int i = tid; i < sb.lq; i += 512)
            if (func_row_meets(p.func, p.func_ld, p.func_n, sb.q0 + i, n0, k1)) {
                qlo = min(qlo, i);
                qhi = max(qhi, i);
            }
        qlo = wave_min(qlo);
        qhi = wave_max(qhi);
        if (lane == 0) {
            q_red[2 * wave] = qlo;
            q_red[2 * wave + 1] = qhi;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            qlo = min(qlo, q_red[2 * w]);
            qhi = max(qhi, q_red[2 * w + 1]);
        }
        // stored dS: row blocks start on multiples of 32 (the extra rows see none of the keys)
        q_begin = qhi >= qlo ? (DS ? qlo & ~31 : qlo) : 0;
        q_end = qhi >= qlo ? qhi + 1 : 0;
    }
    const int ntiles = q_end > q_begin ? (q_end - q_begin + BMQ - 1) / BMQ : 0;
    HSTU_DCHECK(ntiles == 0 || (q_begin >= 0 && q_end <= sb.lq), kDbgTile);
    // func: the words of the tile at rows qt0.. (threads 0-255, one word each: row
    // tid % 64, keys n0 + 32 (tid / 64) ..), in two halves: load_ends reads the
    // row's first endpoints, store_word turns them into the word for slot `slot`
    // (the rest of the endpoints, if any, are read there).
    const int wrow = tid & 63, wkey = n0 + 32 * (tid >> 6);
    auto load_ends = [&](int qt0, int& e0, int& e1, int& e2) {
        e0 = e1 = e2 = 0;
        if constexpr (FUNC) {
            const int i = qt0 + wrow;
            if (tid < 256 && i < sb.lq) {
                HSTU_DCHECK(sb.q0 + i >= 0 && sb.q0 + i < p.func_ld, kDbgFunc);
                e0 = p.func[sb.q0 + i];
                if (p.func_n > 1) {
                    e1 = p.func[(int64_t)p.func_ld + sb.q0 + i];
                    e2 = p.func[2 * (int64_t)p.func_ld + sb.q0 + i];
                }
            }
        }
    };
    auto store_word = [&](int slot, int qt0, int e0, int e1, int e2) {
        if constexpr (FUNC) {
            const int i = qt0 + wrow;
            if (tid < 256)
                fmask[slot * 256 + tid] =
                    i < sb.lq ? func_bits32_pre(e0, e1, e2, p.func, p.func_ld, p.func_n, sb.q0 + i, wkey, sb.lk) : 0u;
        }
    };
    const uint32_t krow = KB + 8192u * kw, vrow = VB + 8192u * kw;

    if (ntiles > 0) {
        // waves 0-3 stage the Q tiles, waves 4-7 the dO tiles
        const bool qgrp = qh == 0;
        const int64_t stok = qgrp ? p.q.tok : p.dout.tok;
        const uint16_t* sbase = qgrp ? p.q.base + (int64_t)sb.q0 * p.q.tok + (int64_t)h * p.q.head
                                     : p.dout.base + (int64_t)sb.q0 * p.dout.tok + (int64_t)h * p.dout.head;
        TileDma<D> dma;
        dma.init(kw, lane, stok);
        if constexpr (D < 32) {
            // columns D..31 of the Q and dO slots are read by the 32-wide transposed blocks
            for (int u = tid; u < 4 * kTileRows * (32 - D) / 8; u += 512) {
                const int sl = u / (kTileRows * (32 - D) / 8), v = u % (kTileRows * (32 - D) / 8);
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        dma.issue(lds0 + (qgrp ? Q0 : D0), sbase, stok, q_begin, sb.lq);
        {
            int e0, e1, e2;
            load_ends(q_begin, e0, e1, e2);
            store_word(0, q_begin, e0, e1, e2);
        }
        wait_global_loads();
        __syncthreads();

        auto step = [&](uint32_t qc, uint32_t dc, uint32_t qn, uint32_t dn, int t) {
            const int qt0 = q_begin + t * BMQ;
            int e0 = 0, e1 = 0, e2 = 0;  // func: the next tile's endpoints, in flight with its DMA
            if (t + 1 < ntiles) {
                dma.issue(lds0 + (qgrp ? qn : dn), sbase, stok, qt0 + BMQ, sb.lq);
                load_ends(qt0 + BMQ, e0, e1, e2);
            }
            const int row0 = qt0 + 32 * qh;
            const uint32_t qr = qc + 8192u * qh, dr = dc + 8192u * qh;
            bool computed = false;  // fused backward: this wave's dS block holds data this step
            auto fq_target = [&](DsOut& ds) {
                ds.on = true;
                ds.lds = lds_addr(fq_ds) + (uint32_t)(qh * 4 + kw) * (2u * kDsBlockElems);
                ds.kcut = key0 + 32 > sb.lk;
                ds.kdead = my_key >= sb.lk;
            };
            if constexpr (FUNC) {
                // the live rows of the block and the wave's live keys decide between
                // skipping it, the unmasked code and the bit-masked code
                if (wave_live && row0 < sb.lq) {
                    const uint32_t wbase = (uint32_t)((t & 1) * 256 + kw * 64 + 32 * qh);
                    const uint32_t word = fmask[wbase + l32];
                    const bool live = row0 + l32 < sb.lq;
                    const uint32_t valid = sb.lk - key0 >= 32 ? ~0u : (1u << (sb.lk - key0)) - 1u;
                    const uint64_t seen = __ballot(live && word != 0);
                    const uint64_t cut = __ballot(live && word != valid);
                    // rows past the sequence (copies of its last row) must be masked out too
                    if (seen != 0) {
                        // stored dS: the block is written exactly when it holds a visible pair,
                        // the test the dq kernel repeats before reading it
                        DsOut ds{nullptr, false, false, false, 0};
                        if constexpr (DS) {
                            ds.on = true;
                            ds.p = ds_base + (ds_rows_before(row0 >> 5, ds_ng, false) + (key0 >> 5)) * kDsBlockElems;
                            HSTU_DCHECK(ds.p >= p.ds && ds.p + kDsBlockElems <= p.ds + (int64_t)p.heads * p.ds_head * kDsBlockElems,
                                        kDbgDs);
                            ds.kcut = key0 + 32 > sb.lk;
                            ds.kdead = my_key >= sb.lk;
                        }
                        if constexpr (FQ) fq_target(ds);
                        computed = true;
                        dkdv_block<D, kBits, FQ>(cut != 0 || row0 + 32 > sb.lq, qr, dr, krow, vrow, qr, dr, dvacc,
                                                 dkacc, roff, toff, row0, 0, 0, g,
                                                 lds_addr(fmask) + 4u * (wbase + 4 * g), ds, p.exp_c, p.alpha);
                    }
                }
            } else {
                // waves whose keys no row of the block sees, or that lie past the sequence, skip it
                const bool run = WINDOW ? row0 + 32 > any_lo && row0 < any_hi : !(CAUSAL && row0 + 31 < key0);
                if (wave_live && run && row0 < sb.lq) {
                    DsOut ds{nullptr, false, false, false, 0};
                    if constexpr (FQ) fq_target(ds);
                    computed = true;
                    if constexpr (DS) {
                        ds.on = true;
                        const int rb = row0 >> 5;
                        const int64_t blk = p.ds_rel >= 0 ? (int64_t)rb * p.ds_kg + (key0 >> 5) - (rb - p.ds_rel)
                                                          : ds_rows_before(rb, ds_ng, p.ds_tri != 0) + (key0 >> 5);
                        ds.p = ds_base + blk * kDsBlockElems;
                        HSTU_DCHECK(ds.p >= p.ds && ds.p + kDsBlockElems <= p.ds + (int64_t)p.heads * p.ds_head * kDsBlockElems,
                                    kDbgDs);
                        ds.kcut = key0 + 32 > sb.lk;
                        ds.kdead = my_key >= sb.lk;
                    }
                    // rows outside those that see every key of the wave, or past the sequence, need the mask
                    dkdv_block<D, kInterval, FQ>(row0 < wlo || row0 + 32 > whi, qr, dr, krow, vrow, qr, dr, dvacc,
                                                 dkacc, roff, toff, row0, lo, hi, g, 0, ds, p.exp_c, p.alpha);
                }
            }
            if constexpr (FQ) {
                // dQ of the tile's rows from its dS blocks and the block's K:
                // dQ^T (32 columns x 32 rows) = K^T dS^T over the block's 128 keys; wave w
                // takes column block w % 4 and row half w / 4, and adds its piece to the
                // fp32 accumulator with atomics (the other key blocks add theirs).
                if (lane == 0) fq_on[qh * 4 + kw] = computed ? 1 : 0;
                __syncthreads();
                const int cb = wave & 3, hq = wave >> 2, rq0 = qt0 + 32 * hq;
                if (32 * cb < DM && rq0 < sb.lq) {
                    const uint2 ko = tr_offsets(32 * cb, lane);
                    const uint2 dtr = ds_tr_offsets(lane);
                    const uint32_t blk0 = lds_addr(fq_ds) + (uint32_t)(hq * 4) * (2u * kDsBlockElems);
                    f32x16 qa = f32x16{};
                    bool any = false;
#pragma unroll
                    for (int s8 = 0; s8 < 8; ++s8) {
                        if (!fq_on[hq * 4 + (s8 >> 1)]) continue;
                        any = true;
                        const uint32_t kaddr = lds0 + KB + 4096u * (uint32_t)s8;
                        const uint32_t daddr = blk0 + (uint32_t)(s8 >> 1) * (2u * kDsBlockElems) +
                                               1024u * (uint32_t)(s8 & 1);
                        qa = mfma32x32x16(ds_read_tr16x2(kaddr + ko.x, kaddr + ko.y),
                                          ds_read_tr16x2(daddr + dtr.x, daddr + dtr.y), qa);
                    }
                    if (any) {
                        // Through LDS (this tile's Q or dO slot, free once every wave has run its
                        // block) into row-major order, so that each atomic instruction covers two
                        // 128-byte row segments instead of 32 rows: lane (l32, g) holds row
                        // ds_pos_row(l32), columns acc_row(r, g); column d of row i sits at
                        // i * 32 + (d ^ ((i >> 1) & 15)) (no bank conflicts either way).
                        const uint32_t tb = lds0 + (qh == 0 ? qc : dc) + 4096u * (uint32_t)kw;
                        // the lane index, opaque to the compiler here, so that the addresses
                        // below are formed in place rather than kept live across the walk
                        int ln = lane;
                        __asm__ volatile("" : "+v"(ln));
                        const int wr = ds_pos_row(ln & 31), gl = ln >> 5;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int d = acc_row(r, gl);
                            *(__attribute__((address_space(3))) float*)(uintptr_t)(
                                tb + 4u * (uint32_t)(wr * 32 + (d ^ ((wr >> 1) & 15)))) = qa[r];
                        }
                        const int d = ln & 31;
                        float* dst = p.dq_acc + ((int64_t)sb.q0 * p.heads + h) * D + 32 * cb + d;
#pragma unroll
                        for (int k2 = 0; k2 < 16; ++k2) {
                            const int i = 2 * k2 + gl;
                            const float x = *(__attribute__((address_space(3))) float*)(uintptr_t)(
                                tb + 4u * (uint32_t)(i * 32 + (d ^ ((i >> 1) & 15))));
                            if (rq0 + i < sb.lq && 32 * cb + d < D) {
                                HSTU_DCHECK(((int64_t)(sb.q0 + rq0 + i) * p.heads + h) * D + 32 * cb + d <
                                                (int64_t)p.total_q * p.heads * D,
                                            kDbgAcc);
                                atomicAdd(dst + (int64_t)(rq0 + i) * p.heads * D, x);
                            }
                        }
                    }
                }
            }
            wait_global_loads();
            // the next tile's words into the other slot, last read before the previous barrier
            if (FUNC && t + 1 < ntiles) store_word((t + 1) & 1, qt0 + BMQ, e0, e1, e2);
            __syncthreads();
        };
        for (int t = 0; t < ntiles; t += 2) {
            step(Q0, D0, Q1, D1, t);
            if (t + 1 < ntiles) step(Q1, D1, Q0, D0, t + 1);
        }
    }

    // add the row-half partial sums: waves 4-7 hand theirs to waves 0-3 through LDS
    __syncthreads();
    constexpr int NREG = DM / 32 * 16;  // accumulator registers per tensor
    const uint32_t red = lds0 + (uint32_t)kw * (2 * NREG * 256) + 4u * lane;
    if (qh == 1) {
#pragma unroll
        for (int db = 0; db < DM / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                *(__attribute__((address_space(3))) float*)(uintptr_t)(red + 256u * (db * 16 + r)) = dvacc[db][r];
                *(__attribute__((address_space(3))) float*)(uintptr_t)(red + 256u * (NREG + db * 16 + r)) = dkacc[db][r];
            }
    }
    __syncthreads();
    if (qh == 1) return;
#pragma unroll
    for (int db = 0; db < DM / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dvacc[db][r] += *(__attribute__((address_space(3))) float*)(uintptr_t)(red + 256u * (db * 16 + r));
            dkacc[db][r] += *(__attribute__((address_space(3))) float*)(uintptr_t)(red + 256u * (NREG + db * 16 + r));
        }

    if (my_key < sb.lk) {
        HSTU_DCHECK((int64_t)sb.k0 + my_key < p.total_k, kDbgRow);
        uint16_t* dk = p.dk.base + (int64_t)(sb.k0 + my_key) * p.dk.tok + (int64_t)h * p.dk.head;
        uint16_t* dv = p.dv.base + (int64_t)(sb.k0 + my_key) * p.dv.tok + (int64_t)h * p.dv.head;
        const float sc = p.out_scale, scv = p.out_scale;
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

// dq from stored dS: one workgroup per (256-row block,
// sequence, head), 8 waves of 32 rows, one workgroup per CU.  Per 64-key tile K
// is staged row-major in LDS (three slots, two tiles ahead, shared by the eight
// waves) and each wave copies its rows' dS blocks into its own LDS ring of three
// slots, also two tiles ahead (both stream from HBM: a one-tile lead left the
// copy latency exposed at every tile), reads its dS^T operands from there and
// accumulates dQ^T += K^T dS^T (A operand: K read transposed).  Both copies are
// direct global->LDS loads that the compiler does not track, so the only waits
// in the loop are the counted ones below.  A wave uses the key groups the dk/dv
// kernel stored for its row block: every group of a sequence's keys without a
// mask, groups G <= R (row block R) under the causal mask; entries outside the
// mask or past the sequence's keys are stored as 0.  Under a token window (left,
// right) row block R uses groups (row0 - left) / 32 .. (row0 + 31 + right) / 32
// (none once row0 - left reaches the sequence's keys), the groups that hold a
// visible pair; the dk/dv kernel wrote each of those (and possibly some blocks of
// zeros besides).  Under the arbitrary mask row block R uses the groups from its
// rows' smallest to their largest visible key, and among those only the groups
// that hold a visible pair (a ballot over its rows' visibility words per tile):
// the blocks the dk/dv kernel computed, and so stored.
template <int D>
__device__ __forceinline__ void dq_ds_tile(uint32_t kt, const uint4 (&dsop)[4],
                                           f32x16 (&acc)[(D < 32 ? 32 : D) / 32],
                                           const uint2 (&toff)[(D < 32 ? 32 : D) / 32]) {
    constexpr int NDB = (D < 32 ? 32 : D) / 32;
    constexpr int NQ = 4 * NDB;  // block kb = i / (2 NDB), step s = i / NDB, column block i % NDB
    constexpr int PF = 4;
    uint4 rd[NQ];
    auto read = [&](int i) {
        if (i < NQ) {
            const int s4 = i / NDB, db = i % NDB;
            rd[i] = ds_read_tr16x2(toff[db].x + kt + 4096 * s4, toff[db].y + kt + 4096 * s4);
        }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) read(i);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        acc[i % NDB] = mfma32x32x16(rd[i], dsop[i / NDB], acc[i % NDB]);
        read(i + PF);
    }
}

// One dS slot of a wave: its two key groups' 32 x 32 blocks as stored, 2 KB each
// (64 bytes per key).
constexpr uint32_t kDsSlotBytes = 2 * 2 * kDsBlockElems;
constexpr int BMD = kDqDsBlockM;  // dq-from-dS kernel: query rows per workgroup (32 per wave)
constexpr int NWD = BMD / 32;     // its waves

template <int D, MaskKind MK>
__global__ __launch_bounds__(512, 1) void bwd_dq_ds_kernel(AttnParams p) {
    constexpr bool CAUSAL = MK == MaskKind::Causal;
    constexpr bool WINDOW = MK == MaskKind::Window;
    constexpr bool FUNC = MK == MaskKind::Func;
    __shared__ int wrange[FUNC ? 2 * 8 : 1];  // func: each wave's key-group range
    constexpr int DM = D < 32 ? 32 : D;
    // [K slots 0-2 | wave 0: dS slots 0-2 | wave 1 | ... | wave 7]
    __shared__ __attribute__((aligned(16))) uint16_t smem[3 * kTileElems + NWD * 3 * kDsSlotBytes / 2];
    const uint32_t lds0 = lds_addr(smem);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    const uint32_t dsl = lds0 + 3 * kTileBytes + (uint32_t)wave * 3 * kDsSlotBytes;

    const int h = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % (unsigned)p.heads));
    BlockItem item;
    const int pidx = (int)(blockIdx.x / (unsigned)p.heads);
    if (!(CAUSAL || MK == MaskKind::None
              ? find_block_by_cost<true>(p.cu_q, p.cu_k, p.batch, p.max_cost, pidx, QueryBlocksGe<BMD, CAUSAL>{p.max_cost}, item)
              : find_block<true>(p.cu_q, p.batch, BMD, p.nblk, pidx, item)))
        return;
    const int b = item.b, m = item.m;
    const SeqBounds sb = seq_bounds(p.cu_q, p.cu_k, b);
    dbg_seq(p, sb, h);
    const int m0 = m * BMD;
    if (m0 >= sb.lq) return;

    const int row0 = m0 + 32 * wave;
    const int my_row = row0 + ds_pos_row(l32);  // the query row of this lane's products
    // Key groups [ga, gb) whose stored dS the wave at row r0 uses (wave-uniform).
    const int gmax = min((sb.lk + 31) >> 5, p.ds_kgr);
    auto groups = [&](int r0, int& ga, int& gb) {
        ga = 0;
        gb = r0 < sb.lq ? gmax : 0;
        if (CAUSAL) gb = min(gb, (r0 >> 5) + 1);
        if (WINDOW) {
            ga = max(0, (r0 - p.win_left) >> 5);
            gb = r0 - p.win_left >= sb.lk ? 0 : min(gb, ((r0 + 31 + p.win_right) >> 5) + 1);
        }
    };
    int gA, gB;
    int wga = 0x7fffffff, wgb = 0;
    int f0 = 0, f1 = 0, f2 = 0;  // func: this lane's row's first endpoints
    if constexpr (FUNC) {
        // the range of the row block's visible keys, reduced over its 32 rows (lanes l
        // and l + 32 hold the same row); inside it, the dk/dv kernel wrote exactly the
        // blocks that hold a visible pair, which the walk tests per tile below
        const int frow = sb.q0 + min(my_row, sb.lq - 1);
        HSTU_DCHECK(frow >= 0 && frow < p.func_ld, kDbgFunc);
        f0 = p.func[frow];
        if (p.func_n > 1) {
            f1 = p.func[(int64_t)p.func_ld + frow];
            f2 = p.func[2 * (int64_t)p.func_ld + frow];
        }
        int rlo = 0x7fffffff, rhi = 0;
        if (my_row < sb.lq) func_key_range(p.func, p.func_ld, p.func_n, sb.q0 + my_row, sb.lk, rlo, rhi);
        func_group_range(wave_min(rlo), wave_max(rhi), gA, gB);
        gB = min(gB, gmax);
        if (lane == 0) {
            wrange[2 * wave] = gA;
            wrange[2 * wave + 1] = gB;
        }
        __syncthreads();
        for (int w = 0; w < NWD; ++w)
            if (wrange[2 * w] < wrange[2 * w + 1]) {
                wga = min(wga, wrange[2 * w]);
                wgb = max(wgb, wrange[2 * w + 1]);
            }
    } else {
        groups(row0, gA, gB);
        // the workgroup walks the 64-key tiles that hold some wave's groups
        for (int w = 0; w < NWD; ++w) {
            int ga, gb;
            groups(m0 + 32 * w, ga, gb);
            if (ga < gb) {
                wga = min(wga, ga);
                wgb = max(wgb, gb);
            }
        }
    }
    gA = __builtin_amdgcn_readfirstlane(gA);
    gB = __builtin_amdgcn_readfirstlane(gB);
    const int t0 = __builtin_amdgcn_readfirstlane(wgb > 0 ? wga >> 1 : 0);
    const int t1 = __builtin_amdgcn_readfirstlane(wgb > 0 ? (wgb + 1) >> 1 : 0);
    const int kv_end = min(sb.lk, 32 * wgb);  // K rows past it only meet zero operands
    // The wave's row block in the workspace, shifted so that group G sits at block
    // G (block 0 when the wave uses none: its copies then fetch in-bounds data that
    // is never used, so that every tile issues the same four copies); each copy moves
    // 1 KB of a block as it is.
    const int64_t seq0 = p.ds_rel >= 0 ? (((int64_t)sb.q0 + 31 * (int64_t)b) >> 5) * p.ds_kg
                                       : ds_seq_base(p.cu_q, p.cu_k, b, p.ds_tri != 0);
    int64_t blk0 = 0;
    if (gA < gB) {
        const int rb = row0 >> 5;
        blk0 = (int64_t)h * p.ds_head + seq0 +
               (p.ds_rel >= 0 ? (int64_t)rb * p.ds_kg - (rb - p.ds_rel)
                              : ds_rows_before(rb, (sb.lk + 31) >> 5, p.ds_tri != 0));
    }
    // the wave's groups [gA, gB) are blocks blk0 + gA .. blk0 + gB - 1
    HSTU_DCHECK(gA >= gB || (blk0 + gA >= 0 && blk0 + gB <= (int64_t)p.heads * p.ds_head), kDbgDs);
    HSTU_DCHECK(t1 == t0 || kv_end <= sb.lk, kDbgTile);
    const uint16_t* dsg = static_cast<const uint16_t*>(uniform_ptr(p.ds + blk0 * kDsBlockElems));
    const uint32_t cpy_off = 16u * (uint32_t)lane;
    auto copy_ds = [&](int t) {
        const uint32_t dst = dsl + (uint32_t)(t % 3) * kDsSlotBytes;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int grp = 2 * t + kb;
            const uint32_t src = grp >= gA && grp < gB ? (uint32_t)grp * (2u * kDsBlockElems) : 0u;  // from dsg
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dma16_lds_stream(dst + (uint32_t)kb * (2u * kDsBlockElems) + 1024u * c, dsg, src + 1024u * c + cpy_off);
        }
    };
    const uint2 dtr = ds_tr_offsets(lane);

    uint2 toff[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
        toff[db] = tr_offsets(32 * db, lane);
        toff[db].x += lds0;
        toff[db].y += lds0;
    }
    f32x16 acc[DM / 32];
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) acc[db] = f32x16{};

    if (t1 > t0) {
        const uint16_t* kbase = p.k.base + (int64_t)sb.k0 * p.k.tok + (int64_t)h * p.k.head;
        TileDma<D, NWD> kdma;  // two 1 KB chunks of each K tile per wave
        kdma.init(wave, lane, p.k.tok);
        if constexpr (D < 32) {
            // columns D..31 of the K slots are read by the 32-wide transposed blocks
            for (int u = tid; u < 3 * kTileRows * (32 - D) / 8; u += 64 * NWD) {
                const int sl = u / (kTileRows * (32 - D) / 8), v = u % (kTileRows * (32 - D) / 8);
                const int r = v / ((32 - D) / 8), c = v % ((32 - D) / 8);
                ds_write16(lds0 + sl * kTileBytes + tile_byte(r, D / 8 + c), make_uint4(0, 0, 0, 0));
            }
        }
        // Issue order: K(0), dS(0), K(1), dS(1), then per tile t: K(t + 2), dS(t + 2)
        // (2 + 4 copies per wave).  After tile t's products, wait until all copies but
        // those of tile t + 2 (if issued) have landed.
        auto wait_copies = [&](int t) {
            if (t < t1) __builtin_amdgcn_s_waitcnt(0x0f76);  // vmcnt(6)
            else __builtin_amdgcn_s_waitcnt(0x0f70);         // vmcnt(0)
        };
        auto kslot = [](int t) { return (uint32_t)(t % 3) * kTileBytes; };
        kdma.issue(lds0 + kslot(t0), kbase, p.k.tok, t0 * BN, kv_end);
        copy_ds(t0);
        if (t0 + 1 < t1) {
            kdma.issue(lds0 + kslot(t0 + 1), kbase, p.k.tok, (t0 + 1) * BN, kv_end);
            copy_ds(t0 + 1);
        }
        wait_copies(t0 + 1);  // K(t0) and dS(t0) have landed
        __syncthreads();

        for (int t = t0; t < t1; ++t) {
            const uint32_t kc = kslot(t);
            if (t + 2 < t1) {
                kdma.issue(lds0 + kslot(t + 2), kbase, p.k.tok, (t + 2) * BN, kv_end);
                copy_ds(t + 2);
            }
            if (2 * t + 1 >= gA && 2 * t < gB) {
                const uint32_t sl = dsl + (uint32_t)(t % 3) * kDsSlotBytes;
                uint4 op[4];
                bool use0 = 2 * t >= gA, use1 = 2 * t + 1 < gB;
                if constexpr (FUNC) {
                    // a group is used only when some row of the block sees one of its keys:
                    // the dk/dv kernel's test for storing the block (others hold no data)
                    const bool live = my_row < sb.lq;
                    const int row = sb.q0 + min(my_row, sb.lq - 1);
                    if (use0)
                        use0 = __ballot(live && func_bits32_pre(f0, f1, f2, p.func, p.func_ld, p.func_n, row, 64 * t,
                                                                sb.lk) != 0u) != 0;
                    if (use1)
                        use1 = __ballot(live && func_bits32_pre(f0, f1, f2, p.func, p.func_ld, p.func_n, row,
                                                                64 * t + 32, sb.lk) != 0u) != 0;
                }
                if (use0) {
                    op[0] = ds_read_tr16x2(sl + dtr.x, sl + dtr.y);
                    op[1] = ds_read_tr16x2(sl + 1024u + dtr.x, sl + 1024u + dtr.y);
                } else {
                    op[0] = op[1] = make_uint4(0, 0, 0, 0);  // the first group is not used
                }
                if (use1) {
                    op[2] = ds_read_tr16x2(sl + 2048u + dtr.x, sl + 2048u + dtr.y);
                    op[3] = ds_read_tr16x2(sl + 3072u + dtr.x, sl + 3072u + dtr.y);
                } else {
                    op[2] = op[3] = make_uint4(0, 0, 0, 0);  // the second group is not used
                }
                dq_ds_tile<D>(kc, op, acc, toff);  // toff holds lds0
            }
            wait_copies(t + 2);
            __syncthreads();
        }
    }

    if (my_row < sb.lq) {
        HSTU_DCHECK((int64_t)sb.q0 + my_row < p.total_q, kDbgRow);
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

template <int D, MaskKind MK>
hipError_t launch_dq_ds(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.items * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_ds_kernel<D, MK>), dim3((unsigned)grid), dim3(64 * NWD), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dq_ds_mask(const AttnParams& p, MaskKind mask, hipStream_t stream) {
    switch (mask) {
        case MaskKind::None: return launch_dq_ds<D, MaskKind::None>(p, stream);
        case MaskKind::Causal: return launch_dq_ds<D, MaskKind::Causal>(p, stream);
        case MaskKind::Window: return launch_dq_ds<D, MaskKind::Window>(p, stream);
        case MaskKind::Func: return launch_dq_ds<D, MaskKind::Func>(p, stream);
    }
}

template <int D, MaskKind MK>
hipError_t launch_dq(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.items * p.heads;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_dq_kernel<D, MK>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, MaskKind MK>
hipError_t launch_dkdv(const AttnParams& p, hipStream_t stream) {
    const int64_t grid = (int64_t)p.items * p.heads;
    if (grid == 0) return hipSuccess;
    if (p.dq_acc != nullptr)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MK, kDkdvFusedDq>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else if (p.ds != nullptr)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MK, kDkdvStoreDs>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MK, kDkdvPlain>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool DKDV>
hipError_t launch_mask(const AttnParams& p, MaskKind mask, hipStream_t stream) {
    switch (mask) {
        case MaskKind::None:
            return DKDV ? launch_dkdv<D, MaskKind::None>(p, stream) : launch_dq<D, MaskKind::None>(p, stream);
        case MaskKind::Causal:
            return DKDV ? launch_dkdv<D, MaskKind::Causal>(p, stream) : launch_dq<D, MaskKind::Causal>(p, stream);
        case MaskKind::Window:
            return DKDV ? launch_dkdv<D, MaskKind::Window>(p, stream) : launch_dq<D, MaskKind::Window>(p, stream);
        case MaskKind::Func:
            return DKDV ? launch_dkdv<D, MaskKind::Func>(p, stream) : launch_dq<D, MaskKind::Func>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <bool DKDV>
hipError_t launch_dir(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream) {
    switch (head_dim) {
        case 16: return launch_mask<16, DKDV>(p, mask, stream);
        case 32: return launch_mask<32, DKDV>(p, mask, stream);
        case 64: return launch_mask<64, DKDV>(p, mask, stream);
        case 128: return launch_mask<128, DKDV>(p, mask, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

#ifdef HSTU_DEBUG
hipError_t debug_take_bwd(uint32_t* out) { return dbg_take(out); }
#endif

hipError_t launch_bwd_dq(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream) {
    return launch_dir<false>(p, head_dim, mask, stream);
}

hipError_t launch_bwd_dkdv(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream) {
    return launch_dir<true>(p, head_dim, mask, stream);
}

// The fused backward's fp32 dQ accumulator: cleared before the dk/dv kernel adds
// into it (a kernel rather than a memset, so the call stays graph-capturable), then
// dQ = (alpha / L_scale) acc rounded to bf16.
__global__ __launch_bounds__(256) void fill_zero_kernel(float4* p, int64_t n4) {
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) p[i] = make_float4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void dq_convert_kernel(const float* acc, TensorOut dq, int64_t rows, int heads,
                                                         int dim, float scale) {
    const int per_row = heads * dim / 4;  // float4 per token
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < rows * per_row; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / per_row;
        const int c = (int)(i % per_row) * 4, hh = c / dim, d = c % dim;
        const float4 v = reinterpret_cast<const float4*>(acc)[i];
        *reinterpret_cast<uint2*>(dq.base + t * dq.tok + hh * dq.head + d) =
            make_uint2(pack_bf16x2(v.x * scale, v.y * scale), pack_bf16x2(v.z * scale, v.w * scale));
    }
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<float4*>(p), n4);
    return hipGetLastError();
}

hipError_t launch_dq_convert(const AttnParams& p, int head_dim, int64_t rows, hipStream_t stream) {
    const int64_t n4 = rows * p.heads * head_dim / 4;
    if (n4 == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(dq_convert_kernel, dim3(grid), dim3(256), 0, stream, p.dq_acc, p.dq, rows, p.heads, head_dim,
                       p.out_scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream) {
    switch (head_dim) {
        case 16: return launch_dq_ds_mask<16>(p, mask, stream);
        case 32: return launch_dq_ds_mask<32>(p, mask, stream);
        case 64: return launch_dq_ds_mask<64>(p, mask, stream);
        case 128: return launch_dq_ds_mask<128>(p, mask, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hstu
