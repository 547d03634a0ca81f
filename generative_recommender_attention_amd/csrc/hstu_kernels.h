// Launch-side view of the HSTU attention kernels: the parameter block every
// kernel takes and the per-direction launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu_device.h"

namespace hstu {

// Mask the kernels are built for.  A token window (left, right) admits key j for
// query i (local indices) iff i - left <= j <= i + right; the host resolves the
// windows that equal full attention or causal to those kinds, and a window side
// with no bound to a bound of max_seqlen_k, which cuts nothing.  Func: each
// packed query row r lists endpoints F0..F_{N-1} (func[n * func_ld + r]) and
// sees the local keys [0, F0) u [F1, F2) u ...
enum class MaskKind : int { None = 0, Causal = 1, Window = 2, Func = 3 };

struct AttnParams {
    const int32_t* cu_q;   // (B + 1) cumulative query lengths, device
    const int32_t* cu_k;   // (B + 1) cumulative key lengths, device
    int32_t batch;         // B
    int32_t heads;         // H
    int32_t total_q;       // T_q, T_k: the token rows of the tensors (bounds tests of debug builds)
    int32_t total_k;
    int32_t nblk;          // row (or key) blocks of the longest sequence
    int32_t items;         // bound on the live blocks: min(nblk B, (T + (block - 1) B) / block);
                           // the grid holds items x heads workgroups
    int32_t max_len;       // max_seqlen_q (forward, dq) or max_seqlen_k (dk/dv): sizes the grid
    int32_t max_cost;      // tiles of the longest walk: ceil(max_seqlen_k / 64) (query-major
                           // kernels) or ceil(max_seqlen_q / 64) (dk/dv), at least 1
    float alpha;           // score scale
    float exp_c;           // -alpha * log2(e), for sig(alpha x) = 1 / (1 + 2^(x exp_c))
    float out_scale;       // alpha / L_scale: the epilogue factor of O, dQ, dK and dV, whose sums
                           // run over raw scores x = q.k (alpha is applied to them in fp32)
    int32_t win_left;      // MaskKind::Window: 0 <= left, right <= max_seqlen_k <= 2^29
    int32_t win_right;
    const int32_t* func;   // MaskKind::Func: endpoints, device, func_n rows of func_ld >= T_q
    int32_t func_n;        // odd, >= 1
    int32_t func_ld;
    TensorRef q, k, v, dout;
    TensorOut o, dq, dk, dv;
    // Backward through stored dS (any mask): the dk/dv kernel writes,
    // and the dS-reading dq kernel reads, bf16 dS in 2 KB blocks of 32 query rows x 32
    // keys; null: the dk/dv kernel writes none.  Block (head h, row block R of batch
    // entry b, key group G) sits at block index h ds_head + ds_block(...) below:
    //  - a window stored relative to R (ds_rel >= 0): ((cu_q[b] + 31 b) / 32 + R) ds_kg
    //    + G - (R - ds_rel): R's groups lie in [R - ds_rel, R - ds_rel + ds_kg);
    //  - otherwise the sequences' blocks are packed one after another (base(b) = the
    //    blocks of the sequences before b), row block after row block, and row block R
    //    keeps the groups it has: min(R + 1, nG) under the causal mask (ds_tri; G <= R),
    //    nG otherwise, nG = ceil(L_k / 32).
    uint16_t* ds;
    int64_t ds_head;       // blocks per head (a bound on every sequence mix the sizes allow)
    int32_t ds_kg;         // window stored relative to R: key-group slots per row block
    int32_t ds_rel;        // ceil(left / 32) for a window stored relative to R, else -1
    int32_t ds_tri;        // 1: causal packing (row block R keeps groups 0..R)
    int32_t ds_kgr;        // key groups the dk/dv grid covers: 4 ceil(max_seqlen_k / 128)
    // Fused backward: fp32 (T_q, H, D) packed dQ accumulator the dk/dv kernel adds
    // each query tile's dQ into with atomics (null: not fused).
    float* dq_acc;
};

// Debug builds: sequence b's token ranges against the totals, and the head.
__device__ __forceinline__ void dbg_seq(const AttnParams& p, const SeqBounds& sb, int h) {
    HSTU_DCHECK(sb.q0 >= 0 && sb.lq >= 0 && (int64_t)sb.q0 + sb.lq <= p.total_q && sb.k0 >= 0 && sb.lk >= 0 &&
                    (int64_t)sb.k0 + sb.lk <= p.total_k,
                kDbgSeq);
    HSTU_DCHECK(h >= 0 && h < p.heads, kDbgHead);
    (void)p;
    (void)sb;
    (void)h;
}

// Elements of one stored dS block (32 x 32 bf16, 2 KB) and of one of its rows.
constexpr int kDsBlockElems = 32 * 32;
constexpr int kDsRowElems = 32;
// Largest byte span of one row block's key groups (4 ceil(max_seqlen_k / 128)
// blocks): the dS-reading dq kernel fetches them by 32-bit byte offsets, so
// max_seqlen_k <= 2^25 (2^32 bytes / 2 KB per 32 keys, less a margin).
constexpr int64_t kMaxDsRowBlockBytes = (int64_t(1) << 32) - 4096;

// Tile shapes (rows per workgroup) used to size the grids.
constexpr int kFwdBlockM = 128;   // query rows per forward / dQ workgroup
constexpr int kBwdBlockN = 128;   // key rows per dK/dV workgroup
constexpr int kDqDsBlockM = 256;  // query rows per workgroup of dQ from stored dS

// Largest token stride (elements) the kernels accept: a 64-row tile spans at
// most 64 strides, addressed by unsigned 32-bit byte offsets.
constexpr int64_t kMaxTokenStride = int64_t(1) << 24;

// Largest max_seqlen_k a window mask accepts: bounds such as i + right + 1, for
// rows i up to a block (128 rows) past the sequence end, stay inside int32.
constexpr int32_t kMaxWindowSeqlen = 1 << 29;

hipError_t launch_fwd(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream);
// dQ from the dS the dk/dv kernel stored (p.ds); mask None, Causal or Window.
hipError_t launch_bwd_dq_ds(const AttnParams& p, int head_dim, MaskKind mask, hipStream_t stream);
// Fused backward: clear n floats (n % 4 == 0, 16-byte aligned); dq = bf16(acc * out_scale)
// for the first `rows` tokens of p.dq_acc (packed (T, H, D) fp32).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
hipError_t launch_dq_convert(const AttnParams& p, int head_dim, int64_t rows, hipStream_t stream);
// `count` one-wave workgroups, each writing {realtime, shader cycles, XCC id, HW_ID}.
hipError_t launch_clock_sample(uint64_t* out, int count, hipStream_t stream);
#ifdef HSTU_DEBUG
// Debug builds: each kernel file's failed-bounds-test word (DebugSite bits), then 0.
hipError_t debug_take_fwd(uint32_t* out);
hipError_t debug_take_bwd(uint32_t* out);
hipError_t debug_take_lmsd(uint32_t* out);
#endif

}  // namespace hstu
