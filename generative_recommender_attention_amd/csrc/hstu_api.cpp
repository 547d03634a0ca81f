// C ABI of libhstu: host-side validation and dispatch.  Declarations and the
// full contract are in include/hstu.h.  Nothing here reads device memory,
// synchronises or allocates; every check is on scalars and pointer values.
#include "hstu.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "hstu_kernels.h"
#include "lmsd_kernels.h"

namespace {

thread_local std::string g_last_error;

hstu_status_t fail(hstu_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

hstu_status_t ok() {
    g_last_error.clear();
    return HSTU_OK;
}

// A tensor operand after stride resolution.
struct Operand {
    const char* name;
    const void* ptr;
    hstu_stride_t stride;
    int64_t rows;  // T of this tensor
};

hstu_status_t check_operand(const hstu_args_t& a, Operand& t) {
    const int64_t H = a.num_heads, D = a.head_dim;
    if (t.stride.token == 0 && t.stride.head == 0) t.stride = hstu_stride_t{H * D, D};
    if (t.rows == 0) return HSTU_OK;  // nothing is read or written through it
    if (t.ptr == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is null", t.name);
    if (reinterpret_cast<uintptr_t>(t.ptr) % 16 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", t.name);
    const int64_t st = t.stride.token, sh = t.stride.head;
    if (st <= 0 || sh <= 0 || st % 8 != 0 || sh % 8 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT,
                    "%s strides (token %lld, head %lld) must be positive multiples of 8 elements", t.name,
                    (long long)st, (long long)sh);
    // Staged tiles are addressed by 32-bit byte offsets from a tile's first row.
    if (st > hstu::kMaxTokenStride)
        return fail(HSTU_ERR_UNSUPPORTED, "%s token stride %lld exceeds %lld elements", t.name, (long long)st,
                    (long long)hstu::kMaxTokenStride);
    // Non-aliasing: either heads nest inside tokens or tokens nest inside heads.
    const bool token_major = sh >= D && (H == 1 || st >= sh * H);
    const bool head_major = st >= D && (t.rows == 1 || sh >= st * t.rows);
    if (!token_major && !head_major)
        return fail(HSTU_ERR_INVALID_ARGUMENT,
                    "%s strides (token %lld, head %lld) map two elements to one address", t.name,
                    (long long)st, (long long)sh);
    return HSTU_OK;
}

// Kernel mask for validated args: the windows (-1, -1) and (-1, 0) run the full
// and causal kernels, which are the same masks.
hstu::MaskKind mask_kind(const hstu_args_t& a) {
    if (a.mask == HSTU_MASK_CAUSAL) return hstu::MaskKind::Causal;
    if (a.mask == HSTU_MASK_FUNC) return hstu::MaskKind::Func;
    if (a.mask != HSTU_MASK_WINDOW) return hstu::MaskKind::None;
    if (a.window_left < 0 && a.window_right < 0) return hstu::MaskKind::None;
    if (a.window_left < 0 && a.window_right == 0) return hstu::MaskKind::Causal;
    return hstu::MaskKind::Window;
}

// Scalar checks common to every entry point; fills the kernel parameter block.
hstu_status_t check_common(const hstu_args_t* a, const int32_t* cu_q, const int32_t* cu_k, hstu::AttnParams& p) {
    if (a == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "args is null");
    if (a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128)
        return fail(HSTU_ERR_UNSUPPORTED, "head_dim %d is not one of 16, 32, 64, 128", a->head_dim);
    if (a->mask != HSTU_MASK_NONE && a->mask != HSTU_MASK_CAUSAL && a->mask != HSTU_MASK_WINDOW &&
        a->mask != HSTU_MASK_FUNC)
        return fail(HSTU_ERR_UNSUPPORTED, "mask %d is not one of HSTU_MASK_NONE, _CAUSAL, _WINDOW, _FUNC", a->mask);
    if (a->mask == HSTU_MASK_WINDOW && (a->window_left < -1 || a->window_right < -1))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "window (%d, %d): bounds must be >= -1", a->window_left,
                    a->window_right);
    if (a->mask == HSTU_MASK_FUNC) {
        if (a->func_n < 1 || a->func_n % 2 != 1)
            return fail(HSTU_ERR_INVALID_ARGUMENT, "func_n %d must be odd and positive", a->func_n);
        if (a->total_q > 0 && a->func_ld < a->total_q)
            return fail(HSTU_ERR_INVALID_ARGUMENT, "func_ld %d < total_q %d", a->func_ld, a->total_q);
        if (a->total_q > 0 && (a->func == nullptr || reinterpret_cast<uintptr_t>(a->func) % 4 != 0))
            return fail(HSTU_ERR_INVALID_ARGUMENT, "func is null or not 4-byte aligned");
    }
    if (a->batch < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "batch %d < 1", a->batch);
    if (a->num_heads < 1) return fail(HSTU_ERR_INVALID_ARGUMENT, "num_heads %d < 1", a->num_heads);
    if (a->total_q < 0 || a->total_k < 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "negative total (total_q %d, total_k %d)", a->total_q, a->total_k);
    if (a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "negative max_seqlen (q %d, k %d)", a->max_seqlen_q,
                    a->max_seqlen_k);
    if (a->max_seqlen_q > a->max_seqlen_k)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "max_seqlen_q %d > max_seqlen_k %d", a->max_seqlen_q,
                    a->max_seqlen_k);
    if (a->max_seqlen_q > a->total_q || a->max_seqlen_k > a->total_k)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "max_seqlen exceeds the total token count");
    if (!std::isfinite(a->alpha)) return fail(HSTU_ERR_INVALID_ARGUMENT, "alpha is not finite");
    if (a->scaling_seqlen < 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "scaling_seqlen %d < 0", a->scaling_seqlen);
    const int32_t ls = a->scaling_seqlen == 0 ? a->max_seqlen_q : a->scaling_seqlen;
    if (ls < 1 && a->total_q > 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "scaling_seqlen resolves to %d; it must be positive", ls);
    if (mask_kind(*a) == hstu::MaskKind::Window && a->max_seqlen_k > hstu::kMaxWindowSeqlen)
        return fail(HSTU_ERR_UNSUPPORTED, "a window mask needs max_seqlen_k <= %d", hstu::kMaxWindowSeqlen);
    if (cu_q == nullptr || cu_k == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "cu_seqlens pointer is null");
    if (reinterpret_cast<uintptr_t>(cu_q) % 4 != 0 || reinterpret_cast<uintptr_t>(cu_k) % 4 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "cu_seqlens pointer is not 4-byte aligned");

    std::memset(&p, 0, sizeof(p));
    p.cu_q = cu_q;
    p.cu_k = cu_k;
    p.batch = a->batch;
    p.heads = a->num_heads;
    p.total_q = a->total_q;
    p.total_k = a->total_k;
    p.alpha = a->alpha;
    p.exp_c = -a->alpha * 1.4426950408889634f;
    p.out_scale = ls >= 1 ? a->alpha / (float)ls : 0.0f;
    if (mask_kind(*a) == hstu::MaskKind::Window) {
        // an unbounded side, or one reaching past every sequence, becomes max_seqlen_k:
        // no row index or key index differs from another by more than that
        auto side = [&](int32_t w) { return w < 0 || w > a->max_seqlen_k ? a->max_seqlen_k : w; };
        p.win_left = side(a->window_left);
        p.win_right = side(a->window_right);
    }
    if (mask_kind(*a) == hstu::MaskKind::Func) {
        p.func = a->func;
        p.func_n = a->func_n;
        p.func_ld = a->func_ld;
    }
    return HSTU_OK;
}

hstu::TensorRef ref(const Operand& t) {
    return hstu::TensorRef{static_cast<const uint16_t*>(t.ptr), t.stride.token, t.stride.head};
}
hstu::TensorOut out(const Operand& t) {
    return hstu::TensorOut{static_cast<uint16_t*>(const_cast<void*>(t.ptr)), t.stride.token, t.stride.head};
}

// Grid of a walk over blocks of `block` rows of the side whose longest sequence
// is max_len and whose tokens number total; the walk's tiles run over the other
// side (longest: other_len).  The live blocks number at most nblk B and at most
// sum_b ceil(L_b / block) <= (total + (block - 1) B) / block.
hstu_status_t set_grid(hstu::AttnParams& p, int32_t max_len, int block, int32_t other_len, int32_t total) {
    const int64_t nblk = ((int64_t)max_len + block - 1) / block;
    const int64_t items = std::min<int64_t>(nblk * p.batch, ((int64_t)total + (int64_t)(block - 1) * p.batch) / block);
    const int64_t grid = items * p.heads;
    if (grid > 0x7fffffffLL)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "problem too large: %lld workgroups", (long long)grid);
    p.nblk = (int32_t)nblk;
    p.items = (int32_t)items;
    p.max_len = max_len;
    p.max_cost = (int32_t)std::max<int64_t>(1, ((int64_t)other_len + 63) / 64);
    return HSTU_OK;
}

hstu_status_t launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

hstu_status_t run_dq(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                     const int32_t* cu_q, const int32_t* cu_k, void* dq, hipStream_t stream) {
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_q, cu_k, p);
    if (st != HSTU_OK) return st;
    Operand ops[] = {{"dout", dout, a->dout, a->total_q}, {"q", q, a->q, a->total_q}, {"k", k, a->k, a->total_k},
                     {"v", v, a->v, a->total_k},          {"dq", dq, a->dq, a->total_q}};
    for (Operand& o : ops)
        if ((st = check_operand(*a, o)) != HSTU_OK) return st;
    p.dout = ref(ops[0]);
    p.q = ref(ops[1]);
    p.k = ref(ops[2]);
    p.v = ref(ops[3]);
    p.dq = out(ops[4]);
    if ((st = set_grid(p, a->max_seqlen_q, hstu::kFwdBlockM, a->max_seqlen_k, a->total_q)) != HSTU_OK) return st;
    if (a->total_q == 0) return ok();
    return launched(hstu::launch_bwd_dq(p, a->head_dim, mask_kind(*a), stream), "hstu_bwd_dq");
}

// Layout of stored dS for validated args (stored = false where the backward always
// recomputes): blocks per head, key-group slots per row block of a window stored
// relative to the row block (rel >= 0: ceil(left / 32), else -1), the causal
// packing flag and the key groups the dk/dv grid covers.
struct DsLayout {
    bool stored;
    int64_t head, kg, kgr;
    int32_t rel;
    bool tri;
};

// Largest sum over sequences of f(n_b), f convex with f(0) = 0, over every batch of at
// most B sequences whose row-block counts n_b = ceil(L_b / 32) satisfy n_b <= nmax and
// sum n_b <= N, N = (T + 31 B) / 32 (sum ceil(L_b / 32) <= sum (L_b + 31) / 32): a convex
// sum is largest at a vertex of that polytope, i.e. k = min(B, N / nmax) sequences of
// nmax row blocks and one of the remainder.
template <class F>
int64_t convex_bound(int64_t T, int64_t B, int64_t maxlen, const F& f) {
    const int64_t N = (T + 31 * B) / 32, nmax = (maxlen + 31) / 32;
    if (nmax == 0) return 0;
    const int64_t k = std::min<int64_t>(B, N / nmax);
    const int64_t r = k < B ? std::min<int64_t>(N - k * nmax, nmax) : 0;
    return k * f(nmax) + f(r);
}

DsLayout ds_layout(const hstu_args_t& a) {
    DsLayout l{false, 0, 0, 0, -1, false};
    const hstu::MaskKind mk = mask_kind(a);
    if (a.total_q == 0 || a.total_k == 0) return l;
    l.kgr = 4 * (((int64_t)a.max_seqlen_k + hstu::kBwdBlockN - 1) / hstu::kBwdBlockN);
    // the dq kernel addresses a row block's groups by 32-bit byte offsets
    if (l.kgr * 2 * hstu::kDsBlockElems > (int64_t)hstu::kMaxDsRowBlockBytes) return l;
    const int64_t B = a.batch, nb = ((int64_t)a.total_q + 31 * B) / 32;
    if (mk == hstu::MaskKind::Window) {
        // row block R (rows 32 R ..) meets key groups R - ceil(left / 32) .. R + floor((31 + right) / 32)
        auto side = [&](int32_t w) { return w < 0 || w > a.max_seqlen_k ? (int64_t)a.max_seqlen_k : (int64_t)w; };
        const int64_t lo = (side(a.window_left) + 31) / 32, hi = (31 + side(a.window_right)) / 32;
        if (lo + hi + 1 < l.kgr) {
            l.kg = lo + hi + 1;
            l.rel = (int32_t)lo;
            l.head = nb * l.kg;  // one slot per row-block slot (cu_q[b] + 31 b) / 32 + R
        }
    }
    if (l.rel < 0 && mk == hstu::MaskKind::Causal) {
        // row block R of a sequence keeps min(R + 1, nG) <= R + 1 groups: at most
        // n (n + 1) / 2 blocks for a sequence of n row blocks
        l.tri = true;
        l.head = convex_bound(a.total_q, B, a.max_seqlen_q, [](int64_t n) { return n * (n + 1) / 2; });
    } else if (l.rel < 0) {
        // every row block keeps nG groups (no mask, a wide window, or the arbitrary mask,
        // whose row blocks use a range of groups not known on the host): nR nG blocks per
        // sequence, and sum_b nR_b nG_b is at most (sum_b nR_b) max nG and (sum_b nG_b) max nR
        const int64_t nq = nb, nk = ((int64_t)a.total_k + 31 * B) / 32;
        l.head = std::min(nq * (((int64_t)a.max_seqlen_k + 31) / 32), nk * (((int64_t)a.max_seqlen_q + 31) / 32));
    }
    // the kernels sum per-sequence block counts in int32
    if (l.head >= (int64_t(1) << 31)) return l;
    l.stored = true;
    return l;
}

// Bytes of stored dS for validated args: 0 where the mask has none (the arbitrary
// mask) or a side has no tokens; else one 2 KB block per (head, row-block slot,
// key-group slot).
hstu_status_t ds_bytes(const hstu_args_t& a, size_t& bytes) {
    bytes = 0;
    const DsLayout l = ds_layout(a);
    if (!l.stored) return HSTU_OK;
    const double approx = (double)a.num_heads * (double)l.head * 2.0 * hstu::kDsBlockElems;
    if (approx > 9.0e18)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "stored dS would need %.3g bytes", approx);
    bytes = (size_t)a.num_heads * (size_t)l.head * 2 * hstu::kDsBlockElems;
    return HSTU_OK;
}

// Checks a dS workspace against the args and points the parameter block at it.
hstu_status_t bind_ds(const hstu_args_t& a, void* ds, size_t ds_bytes_given, hstu::AttnParams& p) {
    if (8 * (((int64_t)a.max_seqlen_k + hstu::kBwdBlockN - 1) / hstu::kBwdBlockN) * hstu::kDsBlockElems >
        (int64_t)hstu::kMaxDsRowBlockBytes)
        return fail(HSTU_ERR_UNSUPPORTED, "stored dS needs max_seqlen_k below 2^25");
    size_t need = 0;
    hstu_status_t st = ds_bytes(a, need);
    if (st != HSTU_OK) return st;
    if (ds_bytes_given < need)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "dS workspace of %zu bytes < %zu needed", ds_bytes_given, need);
    if (need > 0 && (ds == nullptr || reinterpret_cast<uintptr_t>(ds) % 256 != 0))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "dS workspace is null or not 256-byte aligned");
    const DsLayout l = ds_layout(a);
    p.ds = static_cast<uint16_t*>(ds);
    p.ds_head = l.head;
    p.ds_kg = (int32_t)l.kg;
    p.ds_rel = l.rel;
    p.ds_tri = l.tri ? 1 : 0;
    p.ds_kgr = (int32_t)l.kgr;
    return HSTU_OK;
}

// dQ from stored dS: reads k and the workspace only.
hstu_status_t run_dq_ds(const hstu_args_t* a, const void* k, const int32_t* cu_q, const int32_t* cu_k, void* ds,
                        size_t ds_given, void* dq, hipStream_t stream) {
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_q, cu_k, p);
    if (st != HSTU_OK) return st;
    Operand ops[] = {{"k", k, a->k, a->total_k}, {"dq", dq, a->dq, a->total_q}};
    for (Operand& o : ops)
        if ((st = check_operand(*a, o)) != HSTU_OK) return st;
    if ((st = bind_ds(*a, ds, ds_given, p)) != HSTU_OK) return st;
    p.k = ref(ops[0]);
    p.dq = out(ops[1]);
    if ((st = set_grid(p, a->max_seqlen_q, hstu::kDqDsBlockM, a->max_seqlen_k, a->total_q)) != HSTU_OK) return st;
    if (a->total_q == 0) return ok();
    // with no keys the kernel writes dQ = 0 without touching the (empty) workspace
    return launched(hstu::launch_bwd_dq_ds(p, a->head_dim, mask_kind(*a), stream), "hstu_bwd_dq_ds");
}

// dK and dV; with `store_ds`, the kernel also stores dS in the workspace `ds`.
hstu_status_t run_dkdv(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                       const int32_t* cu_q, const int32_t* cu_k, void* dk, void* dv, hipStream_t stream,
                       bool store_ds = false, void* ds = nullptr, size_t ds_given = 0) {
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_q, cu_k, p);
    if (st != HSTU_OK) return st;
    if (store_ds && (st = bind_ds(*a, ds, ds_given, p)) != HSTU_OK) return st;
    Operand ops[] = {{"dout", dout, a->dout, a->total_q}, {"q", q, a->q, a->total_q},
                     {"k", k, a->k, a->total_k},          {"v", v, a->v, a->total_k},
                     {"dk", dk, a->dk, a->total_k},       {"dv", dv, a->dv, a->total_k}};
    for (Operand& o : ops)
        if ((st = check_operand(*a, o)) != HSTU_OK) return st;
    if (a->total_k > 0 && dk == dv) return fail(HSTU_ERR_INVALID_ARGUMENT, "dk and dv are the same buffer");
    p.dout = ref(ops[0]);
    p.q = ref(ops[1]);
    p.k = ref(ops[2]);
    p.v = ref(ops[3]);
    p.dk = out(ops[4]);
    p.dv = out(ops[5]);
    if ((st = set_grid(p, a->max_seqlen_k, hstu::kBwdBlockN, a->max_seqlen_q, a->total_k)) != HSTU_OK) return st;
    if (a->total_k == 0) return ok();
    return launched(hstu::launch_bwd_dkdv(p, a->head_dim, mask_kind(*a), stream),
                    "hstu_bwd_dkdv");
}

}  // namespace

extern "C" {

hstu_status_t hstu_fwd(const hstu_args_t* a, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o, hipStream_t stream) {
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_seqlens_q, cu_seqlens_k, p);
    if (st != HSTU_OK) return st;
    Operand ops[] = {{"q", q, a->q, a->total_q},
                     {"k", k, a->k, a->total_k},
                     {"v", v, a->v, a->total_k},
                     {"o", o, a->o, a->total_q}};
    for (Operand& op : ops)
        if ((st = check_operand(*a, op)) != HSTU_OK) return st;
    p.q = ref(ops[0]);
    p.k = ref(ops[1]);
    p.v = ref(ops[2]);
    p.o = out(ops[3]);
    if ((st = set_grid(p, a->max_seqlen_q, hstu::kFwdBlockM, a->max_seqlen_k, a->total_q)) != HSTU_OK) return st;
    if (a->total_q == 0) return ok();
    return launched(hstu::launch_fwd(p, a->head_dim, mask_kind(*a), stream), "hstu_fwd");
}

hstu_status_t hstu_bwd_dq(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq, hipStream_t stream) {
    return run_dq(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dq, stream);
}

hstu_status_t hstu_bwd_dkdv(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dk, void* dv,
                            hipStream_t stream) {
    return run_dkdv(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dk, dv, stream);
}

hstu_status_t hstu_bwd_dkdv_ds(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dk, void* dv,
                               void* ds, size_t ds_bytes_given, hipStream_t stream) {
    return run_dkdv(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dk, dv, stream, true, ds, ds_bytes_given);
}

hstu_status_t hstu_bwd_dq_ds(const hstu_args_t* a, const void* k, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, const void* ds, size_t ds_bytes_given, void* dq,
                             hipStream_t stream) {
    return run_dq_ds(a, k, cu_seqlens_q, cu_seqlens_k, const_cast<void*>(ds), ds_bytes_given, dq, stream);
}

hstu_status_t hstu_bwd_workspace_size(const hstu_args_t* a, size_t* bytes) {
    if (a == nullptr || bytes == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "args or bytes is null");
    hstu::AttnParams p;
    const int32_t zero[1] = {0};
    hstu_status_t st = check_common(a, zero, zero, p);  // scalar checks only; the pointers are not used
    if (st != HSTU_OK) return st;
    size_t n = 0;
    if ((st = ds_bytes(*a, n)) != HSTU_OK) return st;
    *bytes = n;
    return ok();
}

// Bytes of the fused backward's fp32 dQ accumulator: T_q H D floats, whole 256-byte units.
size_t fused_bytes(const hstu_args_t& a) {
    const size_t n = (size_t)a.total_q * (size_t)a.num_heads * (size_t)a.head_dim * sizeof(float);
    return (n + 255) / 256 * 256;
}

hstu_status_t hstu_bwd_fused_workspace_size(const hstu_args_t* a, size_t* bytes) {
    if (a == nullptr || bytes == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "args or bytes is null");
    hstu::AttnParams p;
    const int32_t zero[1] = {0};
    hstu_status_t st = check_common(a, zero, zero, p);  // scalar checks only
    if (st != HSTU_OK) return st;
    *bytes = fused_bytes(*a);
    return ok();
}

hstu_status_t hstu_bwd_fused(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_seqlens_q, cu_seqlens_k, p);
    if (st != HSTU_OK) return st;
    const size_t need = fused_bytes(*a);
    if (workspace_bytes < need)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (need > 0 && (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is null or not 256-byte aligned");
    Operand ops[] = {{"dout", dout, a->dout, a->total_q}, {"q", q, a->q, a->total_q},
                     {"k", k, a->k, a->total_k},          {"v", v, a->v, a->total_k},
                     {"dq", dq, a->dq, a->total_q},       {"dk", dk, a->dk, a->total_k},
                     {"dv", dv, a->dv, a->total_k}};
    for (Operand& o : ops)
        if ((st = check_operand(*a, o)) != HSTU_OK) return st;
    if (a->total_k > 0 && dk == dv) return fail(HSTU_ERR_INVALID_ARGUMENT, "dk and dv are the same buffer");
    p.dout = ref(ops[0]);
    p.q = ref(ops[1]);
    p.k = ref(ops[2]);
    p.v = ref(ops[3]);
    p.dq = out(ops[4]);
    p.dk = out(ops[5]);
    p.dv = out(ops[6]);
    if ((st = set_grid(p, a->max_seqlen_k, hstu::kBwdBlockN, a->max_seqlen_q, a->total_k)) != HSTU_OK) return st;
    if (a->total_q == 0 && a->total_k == 0) return ok();
    p.dq_acc = static_cast<float*>(workspace);
    const int64_t nacc = (int64_t)a->total_q * a->num_heads * a->head_dim;
    hipError_t e = hstu::launch_fill_zero(p.dq_acc, nacc, stream);
    if (e == hipSuccess && a->total_k > 0) e = hstu::launch_bwd_dkdv(p, a->head_dim, mask_kind(*a), stream);
    if (e == hipSuccess) e = hstu::launch_dq_convert(p, a->head_dim, a->total_q, stream);
    return launched(e, "hstu_bwd_fused");
}

hstu_status_t hstu_bwd(const hstu_args_t* a, const void* dout, const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    // Validate both halves before enqueueing either, so a failure enqueues nothing.
    hstu::AttnParams p;
    hstu_status_t st = check_common(a, cu_seqlens_q, cu_seqlens_k, p);
    if (st != HSTU_OK) return st;
    size_t need = 0;
    if ((st = ds_bytes(*a, need)) != HSTU_OK) return st;
    const bool stored = need > 0 && workspace != nullptr;  // else dQ recomputes the scores
    if (stored && workspace_bytes < need)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (stored && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    Operand ops[] = {{"dout", dout, a->dout, a->total_q}, {"q", q, a->q, a->total_q},
                     {"k", k, a->k, a->total_k},          {"v", v, a->v, a->total_k},
                     {"dq", dq, a->dq, a->total_q},       {"dk", dk, a->dk, a->total_k},
                     {"dv", dv, a->dv, a->total_k}};
    for (Operand& o : ops)
        if ((st = check_operand(*a, o)) != HSTU_OK) return st;
    if (a->total_k > 0 && dk == dv) return fail(HSTU_ERR_INVALID_ARGUMENT, "dk and dv are the same buffer");
    if ((st = set_grid(p, a->max_seqlen_q, hstu::kFwdBlockM, a->max_seqlen_k, a->total_q)) != HSTU_OK) return st;
    if ((st = set_grid(p, a->max_seqlen_k, hstu::kBwdBlockN, a->max_seqlen_q, a->total_k)) != HSTU_OK) return st;
    if (stored) {
        st = run_dkdv(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dk, dv, stream, true, workspace,
                      workspace_bytes);
        if (st != HSTU_OK) return st;
        return run_dq_ds(a, k, cu_seqlens_q, cu_seqlens_k, workspace, workspace_bytes, dq, stream);
    }
    st = run_dq(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dq, stream);
    if (st != HSTU_OK) return st;
    return run_dkdv(a, dout, q, k, v, cu_seqlens_q, cu_seqlens_k, dk, dv, stream);
}

}  // extern "C"

namespace {

// LMSD: scalar checks and the kernel parameter block (pointers filled by the caller).
hstu_status_t lmsd_common(const hstu_lmsd_args_t* a, hstu::LmsdParams& p) {
    if (a == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "args is null");
    if (a->d < 8 || a->d >= 1024 || a->d % 8 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "d %d is not a multiple of 8 in [8, 1024)", a->d);
    if (a->n < 0) return fail(HSTU_ERR_INVALID_ARGUMENT, "n %lld < 0", (long long)a->n);
    if (a->n * (int64_t)a->d > (int64_t(1) << 31))
        return fail(HSTU_ERR_UNSUPPORTED, "n * d exceeds 2^31");
    if (!(a->eps > 0.0f) || !std::isfinite(a->eps)) return fail(HSTU_ERR_INVALID_ARGUMENT, "eps must be positive and finite");
    if (!std::isfinite(a->dropout_ratio) || a->dropout_ratio < 0.0f || a->dropout_ratio >= 1.0f)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "dropout_ratio must be in [0, 1)");
    if (a->dropout_ratio != 0.0f) return fail(HSTU_ERR_UNSUPPORTED, "dropout is not built (dropout_ratio must be 0)");
    std::memset(&p, 0, sizeof(p));
    p.n = a->n;
    p.d = a->d;
    p.segs = 1 + (a->concat_u != 0) + (a->concat_x != 0);
    p.eps = a->eps;
    p.inv_d = 1.0f / (float)a->d;
    p.silu_u = a->apply_u_silu != 0;
    p.concat_u = a->concat_u != 0;
    p.concat_x = a->concat_x != 0;
    return HSTU_OK;
}

// A (rows, d) bf16 matrix with a row stride (0 = packed `packed`).
hstu_status_t lmsd_matrix(const char* name, const void* ptr, int64_t stride, int64_t packed, int64_t width,
                          int64_t rows, int64_t& out) {
    out = stride == 0 ? packed : stride;
    if (rows == 0) return HSTU_OK;
    if (ptr == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is null", name);
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
    if (out < width || out % 8 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "%s row stride %lld must be >= %lld and a multiple of 8", name,
                    (long long)out, (long long)width);
    return HSTU_OK;
}

hstu_status_t lmsd_vector(const char* name, const void* ptr, int64_t align) {
    if (ptr == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is null", name);
    if (reinterpret_cast<uintptr_t>(ptr) % align != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "%s is not %lld-byte aligned", name, (long long)align);
    return HSTU_OK;
}

size_t lmsd_workspace(const hstu_lmsd_args_t* a) {
    if (a->n == 0) return 0;
    const int parts = hstu::lmsd_bwd_parts(a->n, a->d);
    return (size_t)parts * (size_t)a->d * (a->compute_dweight ? 2u : 1u) * sizeof(float);
}

}  // namespace

extern "C" {

hstu_status_t hstu_lmsd_fwd(const hstu_lmsd_args_t* a, const void* x, const void* u, const void* weight,
                            const void* bias, void* y, float* mean, float* rstd, hipStream_t stream) {
    hstu::LmsdParams p;
    hstu_status_t st = lmsd_common(a, p);
    if (st != HSTU_OK) return st;
    if (a->n == 0) return ok();
    int64_t ys;
    if ((st = lmsd_matrix("x", x, a->x_stride, a->d, a->d, a->n, p.x_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("u", u, a->u_stride, a->d, a->d, a->n, p.u_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("y", y, 0, (int64_t)p.segs * a->d, (int64_t)p.segs * a->d, a->n, ys)) != HSTU_OK) return st;
    if ((st = lmsd_vector("weight", weight, 16)) != HSTU_OK) return st;
    if ((st = lmsd_vector("bias", bias, 16)) != HSTU_OK) return st;
    if ((st = lmsd_vector("mean", mean, 4)) != HSTU_OK) return st;
    if ((st = lmsd_vector("rstd", rstd, 4)) != HSTU_OK) return st;
    p.x = static_cast<const uint16_t*>(x);
    p.u = static_cast<const uint16_t*>(u);
    p.weight = static_cast<const uint16_t*>(weight);
    p.bias = static_cast<const uint16_t*>(bias);
    p.y = static_cast<uint16_t*>(y);
    p.mean = mean;
    p.rstd = rstd;
    return launched(hstu::launch_lmsd_fwd(p, stream), "hstu_lmsd_fwd");
}

hstu_status_t hstu_lmsd_bwd_workspace_size(const hstu_lmsd_args_t* a, size_t* bytes) {
    if (bytes == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "bytes is null");
    hstu::LmsdParams p;
    hstu_status_t st = lmsd_common(a, p);
    if (st != HSTU_OK) return st;
    *bytes = lmsd_workspace(a);
    return ok();
}

}  // extern "C"

namespace {

// The LMSD backward on the column-partial buffer `workspace`, from the caller
// (hstu_lmsd_bwd) or the library's own scratch (hstu_lmsd_bwd_noalloc).
hstu_status_t run_lmsd_bwd(const hstu_lmsd_args_t* a, const void* dy, const void* x, const void* u,
                           const void* weight, const void* bias, const float* mean, const float* rstd, void* dx,
                           void* du, void* dweight, void* dbias, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, const char* what) {
    hstu::LmsdParams p;
    hstu_status_t st = lmsd_common(a, p);
    if (st != HSTU_OK) return st;
    const size_t need = lmsd_workspace(a);
    if (workspace_bytes < need)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
    if (need > 0 && (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return fail(HSTU_ERR_INVALID_ARGUMENT, "workspace is null or not 256-byte aligned");
    const int64_t sd = (int64_t)p.segs * a->d;
    if ((st = lmsd_matrix("dy", dy, a->dy_stride, sd, sd, a->n, p.dy_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("x", x, a->x_stride, a->d, a->d, a->n, p.x_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("u", u, a->u_stride, a->d, a->d, a->n, p.u_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("dx", dx, a->dx_stride, a->d, a->d, a->n, p.dx_stride)) != HSTU_OK) return st;
    if ((st = lmsd_matrix("du", du, a->du_stride, a->d, a->d, a->n, p.du_stride)) != HSTU_OK) return st;
    if ((st = lmsd_vector("weight", weight, 16)) != HSTU_OK) return st;
    if ((st = lmsd_vector("bias", bias, 16)) != HSTU_OK) return st;
    if ((st = lmsd_vector("dbias", dbias, 16)) != HSTU_OK) return st;
    if (a->compute_dweight && (st = lmsd_vector("dweight", dweight, 16)) != HSTU_OK) return st;
    if (a->n > 0) {
        if ((st = lmsd_vector("mean", mean, 4)) != HSTU_OK) return st;
        if ((st = lmsd_vector("rstd", rstd, 4)) != HSTU_OK) return st;
    }
    p.dy = static_cast<const uint16_t*>(dy);
    p.x = static_cast<const uint16_t*>(x);
    p.u = static_cast<const uint16_t*>(u);
    p.weight = static_cast<const uint16_t*>(weight);
    p.bias = static_cast<const uint16_t*>(bias);
    p.mean = const_cast<float*>(mean);
    p.rstd = const_cast<float*>(rstd);
    p.dx = static_cast<uint16_t*>(dx);
    p.du = static_cast<uint16_t*>(du);
    p.dweight = a->compute_dweight ? static_cast<uint16_t*>(dweight) : nullptr;
    p.dbias = static_cast<uint16_t*>(dbias);
    p.work = static_cast<float*>(workspace);
    p.part_stride = (int64_t)a->d * (a->compute_dweight ? 2 : 1);
    // no rows: only the column-sum kernel runs, over zero partials, and writes zeros
    return launched(hstu::launch_lmsd_bwd(p, a->n == 0 ? 0 : hstu::lmsd_bwd_parts(a->n, a->d), stream), what);
}

}  // namespace

extern "C" {

hstu_status_t hstu_lmsd_bwd(const hstu_lmsd_args_t* a, const void* dy, const void* x, const void* u,
                            const void* weight, const void* bias, const float* mean, const float* rstd, void* dx,
                            void* du, void* dweight, void* dbias, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    return run_lmsd_bwd(a, dy, x, u, weight, bias, mean, rstd, dx, du, dweight, dbias, workspace, workspace_bytes,
                        stream, "hstu_lmsd_bwd");
}

hstu_status_t hstu_lmsd_bwd_noalloc(const hstu_lmsd_args_t* a, const void* dy, const void* x, const void* u,
                                    const void* weight, const void* bias, const float* mean, const float* rstd,
                                    void* dx, void* du, void* dweight, void* dbias, hipStream_t stream) {
    hstu::LmsdParams p;
    hstu_status_t st = lmsd_common(a, p);
    if (st != HSTU_OK) return st;
    const size_t need = lmsd_workspace(a);
    if (need > hstu::kLmsdScratchBytes)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "the backward needs %zu bytes of scratch; the library holds %zu", need,
                    hstu::kLmsdScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = hstu::lmsd_scratch(&scratch);
    if (e != hipSuccess)
        return fail(HSTU_ERR_DEVICE, "hstu_lmsd_bwd_noalloc: scratch address lookup failed: %s", hipGetErrorString(e));
    return run_lmsd_bwd(a, dy, x, u, weight, bias, mean, rstd, dx, du, dweight, dbias, scratch,
                        hstu::kLmsdScratchBytes, stream, "hstu_lmsd_bwd_noalloc");
}

hstu_status_t hstu_clock_sample(uint64_t* samples, int32_t count, hipStream_t stream) {
    if (count < 1 || count > 65536) return fail(HSTU_ERR_INVALID_ARGUMENT, "count %d is not in [1, 65536]", count);
    if (samples == nullptr || reinterpret_cast<uintptr_t>(samples) % 8 != 0)
        return fail(HSTU_ERR_INVALID_ARGUMENT, "samples is null or not 8-byte aligned");
    return launched(hstu::launch_clock_sample(samples, count, stream), "hstu_clock_sample");
}

hstu_status_t hstu_debug_take(uint32_t* sites) {
    if (sites == nullptr) return fail(HSTU_ERR_INVALID_ARGUMENT, "sites is null");
    *sites = 0;
#ifdef HSTU_DEBUG
    hipError_t e = hipDeviceSynchronize();
    uint32_t w[3] = {0, 0, 0};
    if (e == hipSuccess) e = hstu::debug_take_fwd(&w[0]);
    if (e == hipSuccess) e = hstu::debug_take_bwd(&w[1]);
    if (e == hipSuccess) e = hstu::debug_take_lmsd(&w[2]);
    if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "hstu_debug_take: %s", hipGetErrorString(e));
    *sites = w[0] | w[1] | w[2];
    return ok();
#else
    return fail(HSTU_ERR_UNSUPPORTED, "hstu_debug_take: not a debug build (HSTU_DEBUG)");
#endif
}

const char* hstu_last_error(void) { return g_last_error.c_str(); }

const char* hstu_status_string(hstu_status_t s) {
    switch (s) {
        case HSTU_OK: return "HSTU_OK";
        case HSTU_ERR_INVALID_ARGUMENT: return "HSTU_ERR_INVALID_ARGUMENT";
        case HSTU_ERR_UNSUPPORTED: return "HSTU_ERR_UNSUPPORTED";
        case HSTU_ERR_DEVICE: return "HSTU_ERR_DEVICE";
    }
    return "HSTU_ERR_UNKNOWN";
}

int hstu_abi_version(void) { return HSTU_ABI_VERSION; }

}  // extern "C"
