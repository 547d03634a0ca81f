/*
 * libhstu -- HSTU attention over packed variable-length sequences, for AMD
 * MI355X (gfx950).  C ABI.
 *
 * The operation (HSTU Attention page, "Overview", the four displayed equations):
 * for every packed sequence b and head h,
 *
 *     S = alpha * Q K^T,    A = (M (.) SiLU(S)) / L_scale,    O = A V,
 *
 * with SiLU(s) = s / (1 + exp(-s)), no softmax and no row normalisation, and the
 * heads concatenated.  M is the attention mask inside one sequence; no token
 * ever attends across sequences.  L_scale ("scaling_seqlen") is one positive
 * scalar for the whole call, not a per-sequence token count.
 *
 * Backward (same page, "High-level functions": the backward takes the upstream
 * gradient dO and q, k, v only -- no saved output or statistics -- so the scores
 * are recomputed), by the chain rule on the definition above:
 *
 *     dV = A^T dO
 *     dS = (dO V^T) (.) M (.) SiLU'(S) / L_scale,  SiLU'(s) = sig(s)(1 + s(1 - sig(s)))
 *     dQ = alpha dS K,     dK = alpha dS^T Q
 *
 * -- Tensors ("Tensor layout" table) ------------------------------------------
 *   q, do, o, dq : (T_q, H, D) bf16        k, v, dk, dv : (T_k, H, D) bf16
 *   cu_seqlens_q, cu_seqlens_k : (B + 1) int32, device memory, starting at 0;
 *   sequence b owns rows [cu[b], cu[b+1]).  T_q = cu_seqlens_q[B], T_k likewise.
 *   Every tensor pointer is a device pointer.  Element (t, h, d) of a tensor
 *   lives at base + t * stride.token + h * stride.head + d (in elements): the
 *   last dimension is always contiguous.  A zero stride pair selects the packed
 *   layout (token = H * D, head = D).  Strides must be multiples of 8 elements,
 *   must not map two elements to one address, and base pointers must be 16-byte
 *   aligned ("Tensor layout", the alignment paragraph).  A token stride above
 *   2^24 elements is refused with HSTU_ERR_UNSUPPORTED (tiles of 64 tokens are
 *   addressed with 32-bit byte offsets).  Disjoint views of one
 *   allocation (e.g. dk and dv split from one packed KV gradient buffer) are
 *   fine; overlap between an output and a live input is not checked.
 *
 * -- Masks ("Mask support" table) ---------------------------------------------
 *   The page's window_size = (left, right): key j is visible to query i (both
 *   indices local to the sequence, counted from its first query and first key)
 *   iff i - left <= j <= i + right, where -1 leaves that side unbounded.  This
 *   is the FlashAttention-2 convention, the one the cuDNN SDPA page relates its
 *   diagonal band bounds to (its left bound is our left + 1, its right bound our
 *   right).  The band is aligned top-left; with equal query and key lengths
 *   this is also the bottom-right alignment.
 *   HSTU_MASK_NONE   : window (-1, -1), every key of the sequence is visible.
 *   HSTU_MASK_CAUSAL : window (-1, 0): j <= i.
 *   HSTU_MASK_WINDOW : window (window_left, window_right), each >= -1; a local
 *                      (sliding) window when either side is finite.  (-1, -1)
 *                      and (-1, 0) run exactly as HSTU_MASK_NONE and
 *                      HSTU_MASK_CAUSAL.  Needs max_seqlen_k <= 2^29
 *                      (HSTU_ERR_UNSUPPORTED otherwise).
 *   HSTU_MASK_FUNC   : the arbitrary mask ("Mask support", the func_tensor
 *                      paragraphs).  `func` (device, int32) holds func_n
 *                      endpoint rows of func_ld elements: packed query row r
 *                      (0 <= r < T_q) has endpoints F_n = func[n * func_ld + r],
 *                      n < func_n, func_n odd, and sees the local keys
 *                      [0, F0) u [F1, F2) u [F3, F4) u ... of its sequence.  The
 *                      intervals are independent (they may overlap, come in any
 *                      order, be empty or reach past either end of the
 *                      sequence; keys outside it stay invisible).  The page's
 *                      (1, N, L) tensor with L >= T_q + 256 is func_n = N,
 *                      func_ld = L; only columns below T_q are read, so
 *                      func_ld >= T_q suffices.  The endpoint values are
 *                      trusted and never read on the host; any int32 values are
 *                      safe on the device.  func is read by every kernel of the
 *                      call, so in-place changes between calls are seen.
 *   window_left and window_right are read only with HSTU_MASK_WINDOW, func,
 *   func_n and func_ld only with HSTU_MASK_FUNC.
 *
 * -- Trust and validation ("Tensor layout", the paragraph on metadata) --------
 *   The library checks every scalar and pointer argument on the host and never
 *   reads cu_seqlens on the host, never synchronises and never allocates.  The
 *   values inside cu_seqlens are trusted: they must be non-decreasing, start at
 *   0, end at T_q / T_k, and no sequence may be longer than max_seqlen_q /
 *   max_seqlen_k.  Breaking that contract is undefined behaviour on the device.
 *
 * -- Outputs --------------------------------------------------------------------
 *   Every row r < T_q of o / dq and every row r < T_k of dk / dv is overwritten
 *   (rows with no visible key, or keys no query sees, are written as zeros, the
 *   page's zero-write rule for empty tiles); nothing is read from them first,
 *   and rows past T_q / T_k are not touched.  Caller-owned outputs are the only
 *   outputs: nothing is allocated.
 *
 * -- Execution ------------------------------------------------------------------
 *   Each call validates, enqueues its kernels on `stream` (0 = the null stream)
 *   and returns; results are ready when the stream reaches that point.  Calls
 *   are thread-safe and keep no state between them (two exceptions, stated
 *   where they are declared: hstu_lmsd_bwd_noalloc's per-GPU array, and the
 *   debug build's record of failed bounds tests), so they can be captured in
 *   a HIP graph.  An asynchronous device fault shows up at the caller's next
 *   synchronisation, not in the returned status.  hstu_bwd, on either route,
 *   and its parts are deterministic: the same inputs give bit-identical
 *   gradients; hstu_bwd_fused's dQ is added with atomics in arrival order.
 *
 * -- Errors -----------------------------------------------------------------------
 *   Every entry point returns an hstu_status_t; on failure nothing has been
 *   enqueued and hstu_last_error() returns a message for the calling thread.
 *   No exception, abort or exit ever crosses this interface.
 */
#ifndef LIBHSTU_HSTU_H_
#define LIBHSTU_HSTU_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSTU_ABI_VERSION 7

#if defined(__GNUC__)
#define HSTU_API __attribute__((visibility("default")))
#else
#define HSTU_API
#endif

typedef enum hstu_status {
    HSTU_OK = 0,
    HSTU_ERR_INVALID_ARGUMENT = 1, /* a scalar, pointer, stride or size breaks the contract */
    HSTU_ERR_UNSUPPORTED = 2,      /* head_dim, mask or token stride outside what is built */
    HSTU_ERR_DEVICE = 3            /* the HIP runtime refused a launch                      */
} hstu_status_t;

typedef enum hstu_mask {
    HSTU_MASK_NONE = 0,   /* window (-1, -1) */
    HSTU_MASK_CAUSAL = 1, /* window (-1, 0), top-left aligned */
    HSTU_MASK_WINDOW = 2, /* window (window_left, window_right), top-left aligned */
    HSTU_MASK_FUNC = 3    /* per-row interval list in func (the page's func_tensor) */
} hstu_mask_t;

/* Strides of one (T, H, D) tensor, in elements.  {0, 0} = packed. */
typedef struct hstu_stride {
    int64_t token;
    int64_t head;
} hstu_stride_t;

/* Problem description shared by the forward and the backward (the page asks
 * that both use the same alpha, scaling_seqlen, mask and sequence metadata). */
typedef struct hstu_args {
    int32_t batch;          /* B >= 1; cu_seqlens_q/k hold B + 1 int32 each             */
    int32_t total_q;        /* T_q >= 0: rows of q, do, o, dq                            */
    int32_t total_k;        /* T_k >= 0: rows of k, v, dk, dv                            */
    int32_t num_heads;      /* H >= 1, the same for q, k and v (multi-head only)         */
    int32_t head_dim;       /* D, one of 16, 32, 64, 128                                 */
    int32_t max_seqlen_q;   /* host-known bound on every query length, >= 0              */
    int32_t max_seqlen_k;   /* host-known bound on every key length, >= max_seqlen_q     */
    float alpha;            /* score scale, finite                                        */
    int32_t scaling_seqlen; /* L_scale > 0; 0 selects max_seqlen_q; < 0 is rejected      */
    int32_t mask;           /* an hstu_mask_t                                             */
    int32_t window_left;    /* HSTU_MASK_WINDOW: keys j >= i - window_left; -1 = no bound  */
    int32_t window_right;   /* HSTU_MASK_WINDOW: keys j <= i + window_right; -1 = no bound */
    int32_t func_n;         /* HSTU_MASK_FUNC: endpoints per query row, odd, >= 1          */
    int32_t func_ld;        /* HSTU_MASK_FUNC: elements between endpoint rows, >= T_q       */
    const int32_t* func;    /* HSTU_MASK_FUNC: device, 4-byte aligned, func_n x func_ld     */
    hstu_stride_t q, k, v;  /* input strides                                              */
    hstu_stride_t o;        /* forward output                                             */
    hstu_stride_t dout;     /* backward upstream gradient                                 */
    hstu_stride_t dq, dk, dv; /* backward outputs                                         */
} hstu_args_t;

/* Forward: o = HSTU(q, k, v).  Reads q, k, v, cu_seqlens_q/k; writes o. */
HSTU_API hstu_status_t hstu_fwd(const hstu_args_t* args,
                       const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       void* o, hipStream_t stream);

/* Bytes of device workspace that lets hstu_bwd store dS instead of recomputing
 * the scores for dQ (written to *bytes).  Reads the scalars of `args` only (the
 * pointers in it are not used).  dS (above) is the factor that dQ and dK share;
 * the workspace holds it in bf16 without the 1 / L_scale, which the dQ kernel
 * applies with alpha, in 2 KB blocks of 32 query rows x 32 keys.  A sequence of
 * nR = ceil(L_q / 32) row blocks and nG = ceil(L_k / 32) key groups keeps
 * sum_R min(R + 1, nG) blocks under the causal mask (the lower triangle) and
 * nR nG otherwise; the sequences' blocks are packed one after another, the
 * offsets computed on the device from cu_seqlens.  The size is H times a bound
 * that holds for every length mix the sizes allow, with N_q = (T_q + 31 B) / 32,
 * n = ceil(max_seqlen_q / 32), k = min(B, N_q / n), r = min(N_q - k n, n):
 *   causal:  k n (n + 1) / 2 + r (r + 1) / 2 blocks per head (a sum of
 *            triangles is largest with as many sequences as possible at the
 *            longest length);
 *   no mask: min(N_q ceil(max_seqlen_k / 32), N_k ceil(max_seqlen_q / 32)).
 * A window (left, right) keeps ceil(left / 32) + floor((31 + right) / 32) + 1
 * key-group slots per row-block slot (N_q of them, a side of -1 counting as
 * max_seqlen_k) when that is below 4 ceil(max_seqlen_k / 128), else the no-mask
 * layout; the arbitrary mask uses the no-mask layout (a row block's key groups
 * depend on the endpoints, which the host never reads).  With no tokens on a
 * side, with max_seqlen_k of 2^25 or more or a bound of 2^31 blocks per head or
 * more, it is 0 (those backwards always recompute). */
HSTU_API hstu_status_t hstu_bwd_workspace_size(const hstu_args_t* args, size_t* bytes);

/* Backward, all three gradients.  With a workspace of at least
 * hstu_bwd_workspace_size() bytes (256-byte aligned, caller-owned device
 * memory, contents on entry ignored; the call overwrites it) and a nonzero
 * size, enqueues hstu_bwd_dkdv_ds then hstu_bwd_dq_ds on it; with `workspace` null, or a
 * size of 0, enqueues hstu_bwd_dq then hstu_bwd_dkdv, which need none.  A
 * non-null workspace smaller than the size is HSTU_ERR_INVALID_ARGUMENT.  The
 * two routes round differently (dQ from the bf16 dS of the dk/dv kernel, or
 * from its own recomputed scores) and both meet the same accuracy. */
HSTU_API hstu_status_t hstu_bwd(const hstu_args_t* args, const void* dout,
                       const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward, dQ only (one query-major kernel: recompute S, dS; dQ = alpha dS K). */
HSTU_API hstu_status_t hstu_bwd_dq(const hstu_args_t* args, const void* dout,
                          const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          void* dq, hipStream_t stream);

/* Backward, dK and dV only (one key-major kernel: recompute S, dS;
 * dV = A^T dO, dK = alpha dS^T Q). */
HSTU_API hstu_status_t hstu_bwd_dkdv(const hstu_args_t* args, const void* dout,
                            const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            void* dk, void* dv, hipStream_t stream);

/* hstu_bwd_dkdv that also writes the bf16 dS of every 32 x 32 (rows x keys)
 * block it computes to `ds` (hstu_bwd_workspace_size() bytes, 256-byte aligned;
 * null allowed only when that size is 0), entries outside the mask as 0.  dK
 * and dV are bit-identical to hstu_bwd_dkdv's.  Under the arbitrary mask it
 * writes exactly the blocks that hold a visible pair; the rest of the workspace
 * keeps what it held. */
HSTU_API hstu_status_t hstu_bwd_dkdv_ds(const hstu_args_t* args, const void* dout,
                               const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               void* dk, void* dv, void* ds, size_t ds_bytes,
                               hipStream_t stream);

/* dQ = alpha / L_scale * dS K from the dS that hstu_bwd_dkdv_ds stored in `ds`
 * for the same args and cu_seqlens (enqueue it first on the same stream, or
 * order the two otherwise).  Reads k and ds only (and, under the arbitrary mask,
 * func, to skip the blocks with no visible pair); writes dq.  Any mask, with the
 * same func contents as the hstu_bwd_dkdv_ds call. */
HSTU_API hstu_status_t hstu_bwd_dq_ds(const hstu_args_t* args, const void* k,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             const void* ds, size_t ds_bytes, void* dq,
                             hipStream_t stream);

/* The page's fused backward for D <= 128 ("Current limitations": its backward is
 * not deterministic; Block Sparse Attention page, "Current support", backward:
 * one pass over query x key tiles running all five products, fp32 atomics).  One
 * key-major pass computes dK and dV as hstu_bwd_dkdv does (bit-identical) and,
 * per 64-row query tile, that tile's dQ from its dS and the block's K, added
 * into an fp32 accumulator with atomics; a last kernel writes dq = alpha /
 * L_scale times the sum in bf16.  Three kernels on `stream`: clear the
 * accumulator, the pass, the conversion.  The workspace (caller-owned device
 * memory, 256-byte aligned, hstu_bwd_fused_workspace_size() bytes = T_q H D
 * floats rounded up to 256 bytes, contents on entry ignored) holds the
 * accumulator.  dQ's summation order follows the atomics', so repeated calls
 * may differ in the last bits.  Any mask. */
HSTU_API hstu_status_t hstu_bwd_fused_workspace_size(const hstu_args_t* args, size_t* bytes);
HSTU_API hstu_status_t hstu_bwd_fused(const hstu_args_t* args, const void* dout,
                             const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ==========================================================================
 * HSTU LMSD: LayerNorm, affine, times SiLU(u) (HSTU LMSD page, "Overview").
 *
 * For each of N rows of D values:
 *     mean = sum x / D,  rstd = 1 / sqrt(sum (x - mean)^2 / D + eps),
 *     xh = (x - mean) rstd,  l = xh weight + bias,  a = SiLU(u) or u,
 *     y = [a (if concat_u), x (if concat_x), l a]     (segments of D values)
 * and the page's explicit backward, from dy and the saved mean and rstd:
 *     dl = g a,  da = g l (+ the a segment's gradient),  du = da SiLU'(u) or da,
 *     dx = rstd (dl weight - mean_D(dl weight) - xh mean_D(dl weight xh))
 *          (+ the x segment's gradient),
 *     dweight = sum_rows dl xh,  dbias = sum_rows dl,
 * where g is dy's l a segment.  Dropout is not built: dropout_ratio must be 0
 * (HSTU_ERR_UNSUPPORTED otherwise; the page fixes no random stream that a
 * result could be checked against), so no keep mask is produced or read.
 *
 * Tensors ("Tensor shapes and layouts" table): x, u, dx, du (N, D) bf16 with
 * row strides in elements (0 = D), multiples of 8; weight, bias, dweight, dbias
 * (D) bf16; y (N, S D) bf16 contiguous, S = 1 + concat_u + concat_x; dy (N, S D)
 * bf16 with row stride dy_stride (0 = S D), a multiple of 8; mean, rstd (N)
 * fp32.  All device pointers, 16-byte aligned (mean, rstd: 4-byte).  Limits
 * ("Supported configurations"): N >= 0 with N D <= 2^31, 8 <= D < 1024, D % 8
 * == 0, eps positive and finite.  Outputs must not overlap inputs or each
 * other.  Validation, errors, streams and ownership as for attention above;
 * the backward's workspace (hstu_lmsd_bwd_workspace_size bytes, 256-byte
 * aligned) holds per-workgroup column partials, so dweight and dbias are
 * deterministic.  compute_dweight = 0 skips dweight (its pointer may be null).
 * ========================================================================== */
typedef struct hstu_lmsd_args {
    int64_t n;                /* rows N >= 0                                            */
    int64_t x_stride;         /* row strides in elements; 0 = packed                    */
    int64_t u_stride;
    int64_t dy_stride;        /* 0 = S D                                                */
    int64_t dx_stride;
    int64_t du_stride;
    int32_t d;                /* D: 8 <= D < 1024, D % 8 == 0                           */
    float eps;                /* > 0, finite                                            */
    float dropout_ratio;      /* must be 0                                              */
    int32_t apply_u_silu;     /* nonzero: a = SiLU(u); zero: a = u                      */
    int32_t concat_u;         /* nonzero: y starts with the a segment                   */
    int32_t concat_x;         /* nonzero: y then has the x segment                      */
    int32_t compute_dweight;  /* backward: nonzero computes dweight                     */
} hstu_lmsd_args_t;

/* Forward: y, mean, rstd from x, u, weight, bias. */
HSTU_API hstu_status_t hstu_lmsd_fwd(const hstu_lmsd_args_t* args, const void* x, const void* u,
                            const void* weight, const void* bias, void* y, float* mean, float* rstd,
                            hipStream_t stream);

/* Bytes of device workspace hstu_lmsd_bwd needs (written to *bytes). */
HSTU_API hstu_status_t hstu_lmsd_bwd_workspace_size(const hstu_lmsd_args_t* args, size_t* bytes);

/* Backward: dx, du, dbias and (if compute_dweight) dweight, from dy, the forward's
 * inputs and its saved mean and rstd.  Two kernels on `stream`: rows, then the
 * column sums of the workgroup partials. */
HSTU_API hstu_status_t hstu_lmsd_bwd(const hstu_lmsd_args_t* args, const void* dy, const void* x, const void* u,
                            const void* weight, const void* bias, const float* mean, const float* rstd,
                            void* dx, void* du, void* dweight, void* dbias, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ==========================================================================
 * Measurement helper (not part of the method): enqueues `count` (1..65536)
 * one-wave workgroups on `stream`; workgroup i writes four uint64 values to
 * samples[4 i .. 4 i + 3] (device memory, 8-byte aligned, caller-owned):
 * the 100 MHz real-time counter, the shader-cycle counter (it advances at the
 * shader clock of the XCD it runs on), the XCC id and the HW_ID register.
 * Two such calls around a timed region give each XCD's average shader clock
 * over it.
 * ========================================================================== */
HSTU_API hstu_status_t hstu_clock_sample(uint64_t* samples, int32_t count, hipStream_t stream);

/* hstu_lmsd_bwd for callers that cannot allocate (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the column partials in a scratch array the library holds on
 * each GPU for the life of the process (8,323,072 bytes: 1024 partial rows of
 * 2 x 1016 fp32, the most any valid args need; args needing more, which the D
 * limit rules out, are HSTU_ERR_INVALID_ARGUMENT).  Allocates nothing.  The
 * array is looked up (hipGetSymbolAddress) on a device's first call, with that
 * device current; HSTU_ERR_DEVICE if that fails.  Every call on one GPU shares
 * its array: calls that overlap on one GPU (other streams, other threads, or
 * before an earlier call's kernels finished on another stream) race and give
 * wrong results; calls ordered on one stream do not. */
HSTU_API hstu_status_t hstu_lmsd_bwd_noalloc(const hstu_lmsd_args_t* args, const void* dy, const void* x,
                                    const void* u, const void* weight, const void* bias, const float* mean,
                                    const float* rstd, void* dx, void* du, void* dweight, void* dbias,
                                    hipStream_t stream);

/* ==========================================================================
 * Debug builds (libhstu_debug.so, compiled with -DHSTU_DEBUG): the kernels test
 * every global index they form -- each sequence's token range against T_q and
 * T_k, the head, the rows of each tile copy, load and store, the mask endpoint
 * rows, the stored-dS blocks, the fused dQ accumulator's index, the LMSD rows --
 * and record a failed test as a bit per site (bit 0 sequence bounds, 1 head,
 * 2 load/store row, 3 tile copy rows, 4 endpoint row, 5 stored-dS block,
 * 6 fused-dQ accumulator, 7 LMSD row).  A failed test does not stop the access.
 * hstu_debug_take synchronises the current device, writes the bits recorded
 * since the last call to *sites and clears them.  Release builds write 0 and
 * return HSTU_ERR_UNSUPPORTED.  Not for use while other threads launch work.
 * ========================================================================== */
HSTU_API hstu_status_t hstu_debug_take(uint32_t* sites);

/* Message for the calling thread's last non-OK status ("" if none). */
HSTU_API const char* hstu_last_error(void);

/* Short name of a status code. */
HSTU_API const char* hstu_status_string(hstu_status_t status);

/* HSTU_ABI_VERSION of the built library. */
HSTU_API int hstu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBHSTU_HSTU_H_ */
