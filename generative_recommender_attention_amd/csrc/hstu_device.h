// Device-side building blocks shared by the HSTU attention kernels (gfx950).
//
// Matrix products run on the CDNA4 instruction v_mfma_f32_32x32x16_bf16
// (a 32x32 fp32 tile += 32x16 bf16 * 16x32 bf16, one wavefront of 64 lanes).
// Operand and accumulator placement used throughout, for lane l = 0..63,
// l32 = l % 32 and g = l / 32:
//   A (32 rows x 16 k):  lane holds row l32, k = 8g .. 8g+7   (one 16-byte value)
//   B (16 k x 32 cols):  lane holds col l32, k = 8g .. 8g+7   (one 16-byte value)
//   C (32 x 32, fp32):   lane holds col l32, rows 8(r/4) + 4g + r%4, r = 0..15
// An accumulator C[m][n] keeps its column index in the lane and its row index
// in the register.  The kernels exploit that: the fp32 tile of one product,
// rounded to bf16 in registers, is directly the B operand of the next product
// that contracts over C's row index, with no trip through LDS.  The order of
// the 16 contraction slots is free as long as both operands agree; a B operand
// built from an accumulator takes, for contraction step s (16 rows of C),
// slot t <- row 16s + 4g + (t%4) + 8(t/4), i.e. registers 8(s%2)+t of the
// 32-row block s/2.  The matching A operand is read from a row-major LDS tile
// with the gfx950 transposing read ds_read_b64_tr_b16: within each 16-lane
// group, lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4, i/4+4, i/4+8 and i/4+12, so 16 lanes addressing 4 rows x 16 columns
// receive those 16 columns x 4 rows.  Two such reads give the 8 slots.
//
// LDS tiles: 64 rows of 256 bytes (128 bf16; head dims below 128 leave the
// rest of the row unused).  The 16-byte unit c of row r is stored at unit
// c ^ f(r), f(r) = ((r & 3) << 2) | ((r >> 2) & 3).  With that swizzle both
// access patterns are free of bank conflicts on gfx950's 64-bank LDS (measured
// with SQ_LDS_BANK_CONFLICT): 16-byte row reads by 16 consecutive rows, and
// transposing reads of 4 consecutive rows x 32 bytes by each 16-lane group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// ---- debug builds ----------------------------------------------------------------
// Built with -DHSTU_DEBUG, the kernels test the global indices they form -- each
// sequence's token range against the totals, the head, the rows of every tile copy,
// load and store, the mask endpoint rows, the stored-dS blocks, the fused dQ
// accumulator's index, the LMSD rows -- and a failed test sets its site's bit in a
// device word that each kernel file keeps (dbg_take reads and clears it on the host).
// A failed test neither skips the access nor stops the kernel: a trap would end the
// process on the GPU with no report of where.  Release builds compile the tests out.
enum DebugSite : uint32_t {
    kDbgSeq = 1u << 0,   // a sequence's tokens outside [0, total) (cu_seqlens)
    kDbgHead = 1u << 1,  // a head index outside [0, H)
    kDbgRow = 1u << 2,   // a load or store row outside its sequence or the tensor
    kDbgTile = 1u << 3,  // a tile copy from a first row at or past its valid rows, or past the sequence
    kDbgFunc = 1u << 4,  // an endpoint row outside [0, func_ld)
    kDbgDs = 1u << 5,    // a stored-dS block outside the workspace
    kDbgAcc = 1u << 6,   // a fused-dQ accumulator index outside T_q H D
    kDbgLmsd = 1u << 7,  // an LMSD row or partial row outside its buffer
};
#ifdef HSTU_DEBUG
static __device__ uint32_t dbg_word;
__device__ __forceinline__ void dbg_fail(uint32_t site) {
    __hip_atomic_fetch_or(&dbg_word, site, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#define HSTU_DCHECK(cond, site)                   \
    do {                                          \
        if (!(cond)) ::hstu::dbg_fail(site);      \
    } while (0)
// This file's word, then 0 (the caller has synchronised the device).
static inline hipError_t dbg_take(uint32_t* out) {
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(dbg_word), sizeof(uint32_t));
    const uint32_t zero = 0;
    if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &zero, sizeof(uint32_t));
    return e;
}
#else
#define HSTU_DCHECK(cond, site) \
    do {                        \
    } while (0)
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

constexpr int kTileRows = 64;             // rows per staged LDS tile
constexpr int kRowElems = 128;            // bf16 per LDS tile row (256 bytes)
constexpr int kTileElems = kTileRows * kRowElems;

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

// bf16 B operand from eight consecutive accumulator registers x[0..7].
__device__ __forceinline__ uint4 pack_operand(const float* x) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// ---- swizzled LDS tiles ------------------------------------------------------
__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Element offset of (row r, column d) inside a tile; d % 8 is kept.
__device__ __forceinline__ int tile_off(int r, int d) {
    return r * kRowElems + 8 * ((d >> 3) ^ tile_swz(r)) + (d & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// Wait for this wave's outstanding global loads (including loads into LDS):
// s_waitcnt vmcnt(0), leaving the other counters unconstrained.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// ---- LDS by byte address ------------------------------------------------------
// Kernels that keep all their tiles in one LDS array address them by byte
// offset, so that constant parts (slot, row block, contraction step) fold into
// the instructions' immediate offsets and only a few lane-dependent offsets
// stay in registers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
// The same vector in the global address space: stores through it compile to
// global_store (counted by vmcnt only), where a generic pointer gives flat_store,
// which also counts in lgkmcnt and so holds up every later wait on LDS reads until
// the store has reached memory.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

__device__ __forceinline__ uint4 ds_read16(uint32_t a) {
    const u32x4 v = *(lds_u32x4*)(uintptr_t)a;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void ds_write16(uint32_t a, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    *(lds_u32x4*)(uintptr_t)a = w;
}

// Byte offset of (row r, 16-byte unit c) inside a swizzled tile.
__device__ __forceinline__ uint32_t tile_byte(int r, int c) { return (uint32_t)(r * 256 + 16 * (c ^ tile_swz(r))); }

// Transposing read (see the header comment) from two byte addresses: rows r
// and r + 8 of the same 16-row contraction step.
__device__ __forceinline__ uint4 ds_read_tr16x2(uint32_t lo, uint32_t hi) {
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)lo);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)hi);
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return make_uint4(x.x, x.y, y.x, y.y);
}

// Byte offsets of the transposing reads of lane `lane` for the 32-column block
// starting at column d0, rows 0..15 of a step (add 4096 bytes per further step):
// .x for the rows r, .y for the rows r + 8.
__device__ __forceinline__ uint2 tr_offsets(int d0, int lane) {
    const int grp = lane >> 4, j = lane & 15;
    const int r = 4 * (grp >> 1) + (j >> 2);
    const int d = d0 + 16 * (grp & 1) + 4 * (j & 3);
    return make_uint2((uint32_t)(2 * tile_off(r, d)), (uint32_t)(2 * tile_off(r + 8, d)));
}

// A wave-uniform pointer, asserted to the compiler so that it sits in SGPRs.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One 1 KB global -> LDS copy (global_load_lds_dwordx4, saddr form): lane l
// fetches 16 bytes at gbase + voff and the hardware stores them at LDS byte
// M0 + 16 l.  Issued from inline assembly so that the compiler does not track
// it: it inserts no waits of its own, and the caller orders the copy with
// wait_global_loads() and a barrier.  `lds` and `gbase` must be wave-uniform.
// The compiler's hazard recognizer cannot see that the assembly reads M0 and
// the base SGPRs, so the padding is part of the statement: a vector memory
// instruction that reads an SGPR written by a VALU instruction (the
// v_readfirstlane that moves a base pointer computed in vector registers)
// needs 5 wait states, and an LDS DMA needs 1 after a write of M0; s_nop 4
// gives 5.
__device__ __forceinline__ void dma16_lds(uint32_t lds, const void* gbase, uint32_t voff) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(gbase)));
}
// The same for data read once (streaming, non-temporal cache policy).
__device__ __forceinline__ void dma16_lds_stream(uint32_t lds, const void* gbase, uint32_t voff) {
    __asm__ volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(gbase)));
}

// Staging of one 64-row tile of a (T, H, D) tensor by NW waves with
// dma16_lds: each instruction fills one contiguous 1 KB chunk (4 tile rows),
// lane l writing the 16 bytes at chunk + 16 l; wave w of the NW fills chunks
// w*CPW .. w*CPW + CPW - 1 (CPW = 16 / NW).  The swizzle is applied on the
// global side: lane l fetches the logical unit that belongs at its physical
// slot.  Rows at or past `valid_end` repeat the last valid row, so the data
// stays finite; the kernels mask those rows out.
template <int D, int NW = 4>
struct TileDma {
    static constexpr int CPW = 16 / NW;  // 1 KB chunks per wave
    static_assert(NW * CPW == 16, "a tile is 16 chunks");
    int wave;  // 0 .. NW-1 among the loading waves (wave-uniform)
    int lane;

    __device__ __forceinline__ static int chunk_row(int wave, int i, int lane) { return 4 * (wave * CPW + i) + (lane >> 4); }
    __device__ __forceinline__ static int chunk_col(int r, int lane) { return (lane & 15) ^ tile_swz(r); }

    __device__ __forceinline__ void init(int wave_, int lane_, int64_t) {
        wave = wave_;
        lane = lane_;
    }
    // Fill the tile at LDS byte `tile` with local rows row0 .. row0+63 of the
    // tensor at `base`; rows at or past valid_end repeat row valid_end - 1.  The
    // per-lane source offsets are recomputed at every call (a few VALU
    // instructions) rather than kept in registers across the tile loop: kept,
    // they were among the first values spilled under register pressure, and a
    // reload from scratch between two of these copies made the wave wait for the
    // copy before it.  Offsets fit 32 bits: 2 * (63 tok + 8 * 15) < 2^32 for
    // token strides up to 2^24 elements.
    __device__ __forceinline__ void issue(uint32_t tile, const uint16_t* base, int64_t tok, int row0,
                                          int valid_end) const {
        HSTU_DCHECK(row0 >= 0 && row0 < valid_end, kDbgTile);
        const uint16_t* src = base + (int64_t)row0 * tok;
        const uint32_t dst = tile + (uint32_t)(wave * CPW) * 1024u;
        const int last = row0 + kTileRows <= valid_end ? kTileRows - 1 : valid_end - 1 - row0;
        const uint32_t tok2 = 2u * (uint32_t)tok;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int r = chunk_row(wave, i, lane), c = chunk_col(r, lane);
            if (D == 128 || c < D / 8) dma16_lds(dst + 1024 * i, src, (uint32_t)min(r, last) * tok2 + 16u * (uint32_t)c);
        }
    }
};

// Inclusive prefix sum over the 64 lanes of the wave (all lanes active), on the
// data-parallel-primitive path: shifts by 1, 2, 4, 8 lanes inside each 16-lane
// row, then row 0's and rows 0-1's last lanes broadcast into the rows above.
// Lanes without a source add 0.  Six register moves instead of six dependent
// LDS-crossbar permutes (the searches that number work items run several
// such sums per workgroup before its walk starts).
__device__ __forceinline__ int wave_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
    return v;
}

// Sum of x over the 64 lanes of the wave (all lanes active), wave-uniform.
__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_scan(x), 63); }

// Work-item order for grids over (block, sequence).  Sequence b of length
// L_b = cu[b + 1] - cu[b] has n_b = ceil(L_b / BM) blocks of BM rows.  The live
// blocks are numbered level by level, block index m descending (DESC: for a
// causal mask the query blocks with the most key tiles come first) or ascending
// (the key blocks with the most query tiles come first), and by sequence b
// within a level.  Numbering only the live blocks matters: a workgroup that
// exits at once still holds its place in the dispatcher's in-order queue, and
// runs of such workgroups at the front of a grid were measured to hold back the
// dispatch of the live ones behind them (a quarter of the CU slots in use for
// most of a kernel).  Launching the grid over the host-known bound nblk * B
// leaves the surplus workgroups at the end, where they cost nothing.
//
// Item p -> (b, m), found by the wave without host help: with level l holding
// block index m(l) = DESC ? nblk - 1 - l : l and before(l) the number of live
// blocks on the levels below l, the level is the l with
// before(l) <= p < before(l + 1) (binary search; before is a lane-parallel sum
// over the sequences) and b is the (p - before(l))-th sequence, in order, with
// n_b > m(l).  Every lane returns the same values.  Returns false when p is
// past the last live block.  Each step stays inside [0, B) x [0, nblk), so
// inconsistent metadata cannot send it out of bounds.
struct BlockItem {
    int b, m;
};
template <bool DESC>
__device__ __forceinline__ bool find_block(const int32_t* cu, int B, int BM, int nblk, int p, BlockItem& it) {
    const int lane = threadIdx.x & 63;
    auto nb = [&](int b) { return (cu[b + 1] - cu[b] + BM - 1) / BM; };
    const int n0 = lane < B ? nb(lane) : 0;  // the first 64 sequences stay in a register
    auto below = [&](int n, int l) { return DESC ? max(0, n - (nblk - l)) : min(n, l); };
    auto before = [&](int l) {
        int s = below(n0, l);
        for (int b0 = 64; b0 < B; b0 += 64)
            if (b0 + lane < B) s += below(nb(b0 + lane), l);
        return wave_sum(s);
    };
    if (p >= before(nblk)) return false;
    int lo = 0, hi = nblk;  // before(lo) <= p < before(hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (before(mid) <= p) lo = mid;
        else hi = mid;
    }
    const int m = DESC ? nblk - 1 - lo : lo;
    int k = max(0, p - before(lo));
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int n = b0 == 0 ? n0 : (b0 + lane < B ? nb(b0 + lane) : 0);
        const uint64_t mask = __ballot(n > m);
        const int cnt = __popcll(mask);
        if (k < cnt) {  // then mask has at least k + 1 set bits
            uint64_t mm = mask;
            for (int i = 0; i < k; ++i) mm &= mm - 1;  // drop the k lowest set bits
            it.b = __builtin_amdgcn_readfirstlane(b0 + __builtin_ctzll(mm));
            it.m = __builtin_amdgcn_readfirstlane(m);
            return true;
        }
        k -= cnt;
    }
    return false;
}

// Work-item order by decreasing walk length, for the full and causal masks.
// The workgroup dispatcher of an XCD hands workgroups to its shader engines in
// a fixed rotation and, when the engine whose turn it is has no free CU, waits
// -- even while the other engines have idle CUs.  With items numbered by block
// index (find_block above), walks of very different lengths follow each other
// and one engine fills with long walks while its turn holds back the queue
// (traced on the dk/dv kernel: 208 of the 256 CUs busy for the first half of
// the kernel).  Numbered by decreasing tile count, neighbouring workgroups take
// about as long, the engines drain at the same rate, and the longest walks
// start first.
//
// count_ge(lq, lk, D) is the number of blocks of a sequence with query length
// lq and key length lk whose walk has at least D tiles (every live block counts
// at least 1 tile; none counts more than maxcost); the cost of a sequence's
// blocks must be monotone in the block index, non-decreasing (INC) or
// non-increasing.  Item p -> (b, m): the cost level D is the largest with
// N(D) > p, N(D) = sum over sequences of count_ge(., D) (binary search, a
// lane-parallel sum per step); among the blocks of cost exactly D, ordered by
// sequence, item p is the (p - N(D + 1))-th; within its sequence those blocks
// are a contiguous run of block indices.  Returns false past the last live item.
template <bool INC, class CountGe>
__device__ __forceinline__ bool find_block_by_cost(const int32_t* cu_q, const int32_t* cu_k, int B, int maxcost,
                                                   int p, const CountGe& count_ge, BlockItem& it) {
    const int lane = threadIdx.x & 63;
    auto lens = [&](int b, int& lq, int& lk) {
        lq = lk = 0;
        if (b < B) {
            lq = cu_q[b + 1] - cu_q[b];
            lk = cu_k[b + 1] - cu_k[b];
        }
    };
    int lq0, lk0;  // the first 64 sequences stay in registers
    lens(lane, lq0, lk0);
    auto n_ge = [&](int D) {
        int s = count_ge(lq0, lk0, D);
        for (int b0 = 64; b0 < B; b0 += 64) {
            int a, c;
            lens(b0 + lane, a, c);
            s += count_ge(a, c, D);
        }
        return wave_sum(s);
    };
    if (p >= n_ge(1)) return false;
    int lo = 1, hi = maxcost + 1;  // n_ge(lo) > p >= n_ge(hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (n_ge(mid) > p) lo = mid;
        else hi = mid;
    }
    const int D = lo;
    int k = p - n_ge(D + 1);
    for (int b0 = 0; b0 < B; b0 += 64) {
        int a = lq0, c = lk0;
        if (b0 > 0) lens(b0 + lane, a, c);
        const int all = count_ge(a, c, 1), ge = count_ge(a, c, D), gt = count_ge(a, c, D + 1);
        const int incl = wave_scan(ge - gt);
        const int tot = __builtin_amdgcn_readlane(incl, 63);
        if (k < tot) {
            const int L = __builtin_ctzll(__ballot(incl > k));
            const int before = L > 0 ? __builtin_amdgcn_readlane(incl, L - 1) : 0;
            const int kk = k - before;
            it.b = __builtin_amdgcn_readfirstlane(b0 + L);
            it.m = __builtin_amdgcn_readfirstlane(INC ? __builtin_amdgcn_readlane(all, L) - __builtin_amdgcn_readlane(ge, L) + kk
                                                      : __builtin_amdgcn_readlane(gt, L) + kk);
            return true;
        }
        k -= tot;
    }
    return false;
}

// Blocks of a query-major walk (BM rows per block, 64-key tiles) with at least D
// tiles: causal block m walks min(ceil(lk / 64), (BM / 64)(m + 1)) tiles
// (non-decreasing in m), the full mask ceil(lk / 64) for every block.
template <int BM, bool CAUSAL>
struct QueryBlocksGe {
    int maxcost;
    __device__ __forceinline__ int operator()(int lq, int lk, int D) const {
        const int nb = (lq + BM - 1) / BM;
        if (nb == 0 || D > maxcost) return 0;
        if (D == 1) return nb;
        if (((lk + 63) >> 6) < D) return 0;
        if (!CAUSAL) return nb;
        constexpr int r = BM / 64;
        return nb - min(nb, max(0, (D + r - 1) / r - 1));
    }
};

// Blocks of a key-major walk (BN keys per block, 64-row tiles) with at least D
// tiles: causal block n walks ceil((lq - BN n) / 64) tiles (non-increasing in n),
// the full mask ceil(lq / 64) for every block.
template <int BN, bool CAUSAL>
struct KeyBlocksGe {
    int maxcost;
    __device__ __forceinline__ int operator()(int lq, int lk, int D) const {
        const int nb = (lk + BN - 1) / BN;
        if (nb == 0 || D > maxcost) return 0;
        if (D == 1) return nb;
        if (!CAUSAL) return ((lq + 63) >> 6) >= D ? nb : 0;
        const int x = lq - 64 * (D - 1);  // blocks n with BN n < x
        return x <= 0 ? 0 : min(nb, (x + BN - 1) / BN);
    }
};

// Sequence bounds of batch entry b.
struct SeqBounds {
    int q0, lq, k0, lk;
};
// The values are wave-uniform (b is); saying so keeps them, and the tile base
// pointers derived from them, in scalar registers.
__device__ __forceinline__ SeqBounds seq_bounds(const int32_t* cu_q, const int32_t* cu_k, int b) {
    SeqBounds s;
    s.q0 = __builtin_amdgcn_readfirstlane(cu_q[b]);
    s.lq = __builtin_amdgcn_readfirstlane(cu_q[b + 1]) - s.q0;
    s.k0 = __builtin_amdgcn_readfirstlane(cu_k[b]);
    s.lk = __builtin_amdgcn_readfirstlane(cu_k[b + 1]) - s.k0;
    return s;
}

// sig(alpha x) for a raw score x = q.k (the fp32 MFMA sum of exact bf16
// products): 1 / (1 + 2^(c x)) with c = -alpha log2(e), the scale applied in fp32.
// 2^(c x) overflowing to +inf for large negative alpha x gives exactly 0.
__device__ __forceinline__ float sig_x(float x, float c) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(c * x));
}
// SiLU(alpha x) / alpha = x sig(alpha x); the factor alpha goes into the store.
__device__ __forceinline__ float silu_x(float x, float c) { return x * sig_x(x, c); }

// Marks a branch body the optimizer must not speculate: the mask selects sit
// behind a uniform branch so that interior tiles skip them, and an if-converted
// (always executed) version would cost two VALU instructions per score.
__device__ __forceinline__ void keep_branch() { __asm__ volatile(""); }

// ---- interval-list masks -------------------------------------------------------
// Bits of the W keys n0 .. n0 + W - 1 (W = 32 or 64; bit k is key n0 + k) that the
// interval [a, b) covers.  Any int32 endpoints are safe: differences are taken
// only where they cannot overflow.
__device__ __forceinline__ uint64_t span_bits64(int a, int b, int n0) {
    const int lo = a <= n0 ? 0 : min(a - n0, 64);
    const int hi = b <= n0 ? 0 : min(b - n0, 64);
    if (hi <= lo) return 0;
    const uint64_t below_hi = hi >= 64 ? ~0ull : (1ull << hi) - 1;
    return below_hi & ~((1ull << lo) - 1);
}
__device__ __forceinline__ uint32_t span_bits32(int a, int b, int n0) {
    const int lo = a <= n0 ? 0 : min(a - n0, 32);
    const int hi = b <= n0 ? 0 : min(b - n0, 32);
    if (hi <= lo) return 0;
    const uint32_t below_hi = hi >= 32 ? ~0u : (1u << hi) - 1;
    return below_hi & ~((1u << lo) - 1);
}

// Visible keys of packed query row `row` among local keys n0 .. n0 + 63 of a
// sequence with lk keys, for endpoints f[n * ld + row], n < N (N odd):
// [0, F0) u [F1, F2) u ... , cut to [0, lk).
__device__ __forceinline__ uint64_t func_bits64(const int32_t* f, int ld, int N, int row, int n0, int lk) {
    HSTU_DCHECK(row >= 0 && row < ld, kDbgFunc);
    uint64_t m = span_bits64(0, f[row], n0);
    for (int n = 1; n + 1 < N; n += 2)
        m |= span_bits64(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row], n0);
    return m & span_bits64(0, lk, n0);
}
__device__ __forceinline__ uint32_t func_bits32(const int32_t* f, int ld, int N, int row, int n0, int lk) {
    HSTU_DCHECK(row >= 0 && row < ld, kDbgFunc);
    uint32_t m = span_bits32(0, f[row], n0);
    for (int n = 1; n + 1 < N; n += 2)
        m |= span_bits32(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row], n0);
    return m & span_bits32(0, lk, n0);
}

// The same, with the row's first three endpoints already in registers (f0; f1, f2
// when N > 1): only endpoints past the third are read from memory.
__device__ __forceinline__ uint64_t func_bits64_pre(int f0, int f1, int f2, const int32_t* f, int ld, int N, int row,
                                                    int n0, int lk) {
    HSTU_DCHECK(N <= 3 || (row >= 0 && row < ld), kDbgFunc);
    uint64_t m = span_bits64(0, f0, n0);
    if (N > 1) m |= span_bits64(f1, f2, n0);
    for (int n = 3; n + 1 < N; n += 2)
        m |= span_bits64(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row], n0);
    return m & span_bits64(0, lk, n0);
}
__device__ __forceinline__ uint32_t func_bits32_pre(int f0, int f1, int f2, const int32_t* f, int ld, int N, int row,
                                                    int n0, int lk) {
    HSTU_DCHECK(N <= 3 || (row >= 0 && row < ld), kDbgFunc);
    uint32_t m = span_bits32(0, f0, n0);
    if (N > 1) m |= span_bits32(f1, f2, n0);
    for (int n = 3; n + 1 < N; n += 2)
        m |= span_bits32(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row], n0);
    return m & span_bits32(0, lk, n0);
}

// Smallest and one past the largest visible key of row `row` (lo >= hi: none).
__device__ __forceinline__ void func_key_range(const int32_t* f, int ld, int N, int row, int lk, int& lo, int& hi) {
    HSTU_DCHECK(row >= 0 && row < ld, kDbgFunc);
    lo = 0x7fffffff;
    hi = 0;
    auto add = [&](int a, int b) {
        a = max(a, 0);
        b = min(b, lk);
        if (b > a) {
            lo = min(lo, a);
            hi = max(hi, b);
        }
    };
    add(0, f[row]);
    for (int n = 1; n + 1 < N; n += 2) add(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row]);
}

// func_key_range with the row's first three endpoints already in registers.
__device__ __forceinline__ void func_key_range_pre(int f0, int f1, int f2, const int32_t* f, int ld, int N, int row,
                                                   int lk, int& lo, int& hi) {
    HSTU_DCHECK(N <= 3 || (row >= 0 && row < ld), kDbgFunc);
    lo = 0x7fffffff;
    hi = 0;
    auto add = [&](int a, int b) {
        a = max(a, 0);
        b = min(b, lk);
        if (b > a) {
            lo = min(lo, a);
            hi = max(hi, b);
        }
    };
    add(0, f0);
    if (N > 1) add(f1, f2);
    for (int n = 3; n + 1 < N; n += 2) add(f[(int64_t)n * ld + row], f[(int64_t)(n + 1) * ld + row]);
}

// Whether row `row` sees any key of [k0, k1) (0 <= k0, k1 <= lk).
__device__ __forceinline__ bool func_row_meets(const int32_t* f, int ld, int N, int row, int k0, int k1) {
    HSTU_DCHECK(row >= 0 && row < ld, kDbgFunc);
    bool hit = min(f[row], k1) > k0;
    for (int n = 1; n + 1 < N; n += 2)
        hit |= min(f[(int64_t)(n + 1) * ld + row], k1) > max(f[(int64_t)n * ld + row], k0);
    return hit;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
}
// The same over each half of the wave (lanes 0-31 and 32-63 separately).
__device__ __forceinline__ int half_wave_min(int x) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ int half_wave_max(int x) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return x;
}

// Stored dS under the arbitrary mask: the key groups [ga, gb) of a 32-row block are
// those from the smallest to the largest visible key of any of its rows, from the
// block's reduced [lo, hi) (lo >= hi: no visible key, no groups).  The dk/dv kernel
// writes every block of that range (those no visible pair falls in as zeros) and the
// dq kernel reads exactly those, both reducing the same rows.
__device__ __forceinline__ void func_group_range(int lo, int hi, int& ga, int& gb) {
    ga = lo < hi ? lo >> 5 : 0;
    gb = lo < hi ? (hi + 31) >> 5 : 0;
}

// ---- stored dS layout ----------------------------------------------------------
// Blocks (32 rows x 32 keys) of stored dS that row blocks 0 .. R - 1 of a sequence
// with nG key groups keep: row block R' keeps min(R' + 1, nG) of them under the
// causal mask (tri), nG otherwise.  With R = the sequence's row-block count it is
// the sequence's whole share.
__device__ __forceinline__ int64_t ds_rows_before(int R, int nG, bool tri) {
    const int64_t r = R, n = nG;
    if (!tri) return r * n;
    return r <= n ? r * (r + 1) / 2 : n * (n + 1) / 2 + (r - n) * n;
}

// Blocks of stored dS of the sequences before batch entry b (wave-uniform b; every
// lane returns the same value): a lane-parallel sum over the sequences, 64 at a
// time.  Each sum fits int32: the host sizes the workspace by a bound on the total
// below 2^31 blocks per head.
__device__ __forceinline__ int64_t ds_seq_base(const int32_t* cu_q, const int32_t* cu_k, int b, bool tri) {
    const int lane = threadIdx.x & 63;
    int64_t acc = 0;
    for (int b0 = 0; b0 < b; b0 += 64) {
        const int bb = b0 + lane;
        int cnt = 0;
        if (bb < b) {
            const int nR = (cu_q[bb + 1] - cu_q[bb] + 31) >> 5, nG = (cu_k[bb + 1] - cu_k[bb] + 31) >> 5;
            cnt = (int)ds_rows_before(nR, nG, tri);
        }
        acc += wave_sum(cnt);
    }
    return acc;
}

// Row of accumulator register r (0..15) inside a 32-row block, for lane half g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

}  // namespace hstu
