// Host-side check of libhstu's C ABI and of the CPU oracle, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  No GPU is
// used: every library call below is built to fail validation before anything
// is enqueued (or has nothing to enqueue), and the oracle runs on small inputs.
// Exit status 0 and no sanitizer report means every check passed.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "hstu.h"

extern "C" {
int oracle_hstu_fwd(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D, const double* q,
                    const double* k, const double* v, double alpha, double ls, int64_t left, int64_t right,
                    const int32_t* func, int64_t func_n, int64_t func_ld, const int64_t* rows, int64_t nrows,
                    double* out);
int oracle_hstu_bwd_dq(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D, const double* dout,
                       const double* q, const double* k, const double* v, double alpha, double ls, int64_t left,
                       int64_t right, const int32_t* func, int64_t func_n, int64_t func_ld, const int64_t* rows,
                       int64_t nrows, double* out);
int oracle_hstu_bwd_dkdv(int64_t B, const int32_t* cu_q, const int32_t* cu_k, int64_t H, int64_t D,
                         const double* dout, const double* q, const double* k, const double* v, double alpha,
                         double ls, int64_t left, int64_t right, const int32_t* func, int64_t func_n,
                         int64_t func_ld, const int64_t* rows, int64_t nrows, double* dk, double* dv);
void oracle_lmsd_fwd(int64_t n, int64_t d, const double* x, int64_t xs, const double* u, int64_t us, const double* w,
                     const double* b, double eps, int silu_u, int concat_u, int concat_x, double* y, double* mean,
                     double* rstd);
void oracle_lmsd_bwd(int64_t n, int64_t d, const double* dy, int64_t dys, const double* x, int64_t xs,
                     const double* u, int64_t us, const double* w, const double* b, const double* mean,
                     const double* rstd, int silu_u, int concat_u, int concat_x, double* dx, double* du, double* dw,
                     double* db);
}

namespace {

int g_failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, hstu_last_error());
        ++g_failures;
    }
}

// Addresses that are never dereferenced: every call that receives them fails
// host validation first.
void* const FAKE = reinterpret_cast<void*>(uintptr_t(0x100000));
void* fake(uintptr_t off) { return reinterpret_cast<void*>(uintptr_t(0x100000) + off); }

hstu_args_t good() {
    hstu_args_t a;
    std::memset(&a, 0, sizeof(a));
    a.batch = 2;
    a.total_q = a.total_k = 32;
    a.num_heads = 2;
    a.head_dim = 64;
    a.max_seqlen_q = a.max_seqlen_k = 20;
    a.alpha = 0.125f;
    a.mask = HSTU_MASK_CAUSAL;
    return a;
}

hstu_status_t fwd(const hstu_args_t& a, void* q = FAKE, void* o = FAKE, void* cu = FAKE) {
    return hstu_fwd(&a, q, FAKE, FAKE, static_cast<const int32_t*>(cu), static_cast<const int32_t*>(FAKE), o, nullptr);
}

void check_rejections() {
    struct Case {
        const char* what;
        void (*edit)(hstu_args_t&);
        hstu_status_t want;
    };
    const Case cases[] = {
        {"head_dim 48", [](hstu_args_t& a) { a.head_dim = 48; }, HSTU_ERR_UNSUPPORTED},
        {"head_dim 256", [](hstu_args_t& a) { a.head_dim = 256; }, HSTU_ERR_UNSUPPORTED},
        {"mask 4", [](hstu_args_t& a) { a.mask = 4; }, HSTU_ERR_UNSUPPORTED},
        {"func_n even", [](hstu_args_t& a) { a.mask = HSTU_MASK_FUNC; a.func_n = 2; a.func_ld = 32; a.func = (const int32_t*)FAKE; }, HSTU_ERR_INVALID_ARGUMENT},
        {"func_ld short", [](hstu_args_t& a) { a.mask = HSTU_MASK_FUNC; a.func_n = 3; a.func_ld = 31; a.func = (const int32_t*)FAKE; }, HSTU_ERR_INVALID_ARGUMENT},
        {"func null", [](hstu_args_t& a) { a.mask = HSTU_MASK_FUNC; a.func_n = 3; a.func_ld = 32; a.func = nullptr; }, HSTU_ERR_INVALID_ARGUMENT},
        {"window -2", [](hstu_args_t& a) { a.mask = HSTU_MASK_WINDOW; a.window_left = -2; }, HSTU_ERR_INVALID_ARGUMENT},
        {"window past 2^29", [](hstu_args_t& a) { a.mask = HSTU_MASK_WINDOW; a.window_left = 8; a.total_q = a.total_k = (1 << 29) + 2; a.max_seqlen_k = (1 << 29) + 1; }, HSTU_ERR_UNSUPPORTED},
        {"batch 0", [](hstu_args_t& a) { a.batch = 0; }, HSTU_ERR_INVALID_ARGUMENT},
        {"heads 0", [](hstu_args_t& a) { a.num_heads = 0; }, HSTU_ERR_INVALID_ARGUMENT},
        {"negative total", [](hstu_args_t& a) { a.total_q = -1; }, HSTU_ERR_INVALID_ARGUMENT},
        {"max_q > max_k", [](hstu_args_t& a) { a.max_seqlen_q = 21; }, HSTU_ERR_INVALID_ARGUMENT},
        {"max above total", [](hstu_args_t& a) { a.max_seqlen_q = a.max_seqlen_k = 40; }, HSTU_ERR_INVALID_ARGUMENT},
        {"scaling < 0", [](hstu_args_t& a) { a.scaling_seqlen = -1; }, HSTU_ERR_INVALID_ARGUMENT},
        {"scaling resolves to 0", [](hstu_args_t& a) { a.max_seqlen_q = 0; }, HSTU_ERR_INVALID_ARGUMENT},
        {"alpha inf", [](hstu_args_t& a) { a.alpha = INFINITY; }, HSTU_ERR_INVALID_ARGUMENT},
        {"alpha nan", [](hstu_args_t& a) { a.alpha = NAN; }, HSTU_ERR_INVALID_ARGUMENT},
        {"token stride too large", [](hstu_args_t& a) { a.k.token = (int64_t(1) << 24) + 8; a.k.head = 64; }, HSTU_ERR_UNSUPPORTED},
        {"aliasing strides", [](hstu_args_t& a) { a.q.token = 64; a.q.head = 8; }, HSTU_ERR_INVALID_ARGUMENT},
    };
    for (const Case& c : cases) {
        hstu_args_t a = good();
        c.edit(a);
        const hstu_status_t st = fwd(a);
        expect(st == c.want, c.what);
        expect(std::strlen(hstu_last_error()) > 0, c.what);
        std::string msg = hstu_status_string(st);
        expect(!msg.empty(), "status string");
    }
    hstu_args_t a = good();
    expect(fwd(a, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "q null");
    expect(fwd(a, FAKE, fake(8)) == HSTU_ERR_INVALID_ARGUMENT, "o misaligned");
    expect(fwd(a, FAKE, FAKE, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "cu null");
    expect(hstu_fwd(nullptr, FAKE, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE, FAKE, nullptr) ==
               HSTU_ERR_INVALID_ARGUMENT, "args null");
    hstu_args_t empty = good();
    empty.total_q = 0;
    empty.max_seqlen_q = 0;
    empty.scaling_seqlen = 4;
    expect(fwd(empty) == HSTU_OK, "no queries: nothing to enqueue");

    // backward
    const int32_t* cu = static_cast<const int32_t*>(FAKE);
    expect(hstu_bwd(&a, FAKE, FAKE, FAKE, FAKE, cu, cu, FAKE, FAKE, FAKE, nullptr, 0, nullptr) ==
               HSTU_ERR_INVALID_ARGUMENT, "dk == dv");
    expect(hstu_bwd_dq(&a, nullptr, FAKE, FAKE, FAKE, cu, cu, FAKE, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "dout null");
    size_t ws = 0;
    expect(hstu_bwd_workspace_size(&a, &ws) == HSTU_OK && ws > 0, "workspace size");
    expect(hstu_bwd(&a, FAKE, FAKE, FAKE, FAKE, cu, cu, FAKE, fake(16), fake(32), fake(4096), ws - 1, nullptr) ==
               HSTU_ERR_INVALID_ARGUMENT, "workspace too small");
    expect(hstu_bwd_dkdv_ds(&a, FAKE, FAKE, FAKE, FAKE, cu, cu, FAKE, fake(16), nullptr, ws, nullptr) ==
               HSTU_ERR_INVALID_ARGUMENT, "dS workspace null");
    expect(hstu_bwd_dq_ds(&a, FAKE, cu, cu, fake(128), ws, FAKE, nullptr) == HSTU_ERR_INVALID_ARGUMENT,
           "dS workspace misaligned");
    expect(hstu_bwd_workspace_size(nullptr, &ws) == HSTU_ERR_INVALID_ARGUMENT, "workspace args null");
    expect(hstu_bwd_fused_workspace_size(&a, &ws) == HSTU_OK && ws == 32 * 2 * 64 * 4, "fused workspace size");
    expect(hstu_bwd_fused(&a, FAKE, FAKE, FAKE, FAKE, cu, cu, FAKE, fake(16), fake(32), fake(4096), ws - 4,
                          nullptr) == HSTU_ERR_INVALID_ARGUMENT, "fused workspace too small");
    expect(hstu_clock_sample(nullptr, 4, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "clock null");
    expect(hstu_clock_sample(static_cast<uint64_t*>(FAKE), 0, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "clock count");

    // workspace sizes over many argument sets: a whole number of 2 KB blocks per head
    std::mt19937 rng(5);
    for (int i = 0; i < 20000; ++i) {
        hstu_args_t r = good();
        r.batch = 1 + (int)(rng() % 200);
        r.max_seqlen_k = 1 + (int)(rng() % 20000);
        r.max_seqlen_q = 1 + (int)(rng() % r.max_seqlen_k);
        r.total_k = r.max_seqlen_k + (int)(rng() % 100000);
        r.total_q = r.max_seqlen_q + (int)(rng() % 100000);
        r.num_heads = 1 + (int)(rng() % 16);
        r.head_dim = 16 << (rng() % 4);
        r.mask = (int)(rng() % 4);
        r.window_left = (int)(rng() % 3000) - 1;
        r.window_right = (int)(rng() % 3000) - 1;
        r.func_n = 3;
        r.func_ld = r.total_q;
        r.func = static_cast<const int32_t*>(FAKE);
        size_t n = 0;
        const hstu_status_t st = hstu_bwd_workspace_size(&r, &n);
        expect(st == HSTU_OK || st == HSTU_ERR_UNSUPPORTED, "workspace size status");
        if (st == HSTU_OK) expect(n % (2048 * (size_t)r.num_heads) == 0, "workspace size is whole blocks per head");
    }

    // LMSD
    hstu_lmsd_args_t l;
    std::memset(&l, 0, sizeof(l));
    l.n = 10;
    l.d = 64;
    l.eps = 1e-6f;
    l.apply_u_silu = l.concat_u = l.concat_x = l.compute_dweight = 1;
    hstu_lmsd_args_t bad = l;
    bad.d = 12;
    expect(hstu_lmsd_fwd(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, nullptr) ==
               HSTU_ERR_UNSUPPORTED, "lmsd d 12");
    bad = l;
    bad.dropout_ratio = 0.1f;
    expect(hstu_lmsd_fwd(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, nullptr) ==
               HSTU_ERR_UNSUPPORTED, "lmsd dropout");
    expect(hstu_lmsd_fwd(&l, nullptr, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, nullptr) ==
               HSTU_ERR_INVALID_ARGUMENT, "lmsd x null");
    expect(hstu_lmsd_bwd_workspace_size(&l, &ws) == HSTU_OK && ws > 0, "lmsd workspace");
    expect(hstu_lmsd_bwd(&l, FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, FAKE, FAKE, FAKE, FAKE,
                         nullptr, ws, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "lmsd workspace null");
    bad = l;
    bad.eps = 0.0f;
    expect(hstu_lmsd_bwd_noalloc(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE, (float*)FAKE, FAKE, FAKE, FAKE,
                                 FAKE, nullptr) == HSTU_ERR_INVALID_ARGUMENT, "lmsd noalloc eps");
    expect(hstu_abi_version() == HSTU_ABI_VERSION, "abi version");
}

// The oracle on small problems with every mask form, every row and a subset of rows.
void check_oracle() {
    std::mt19937 rng(7);
    std::normal_distribution<double> nd(0.0, 1.0);
    for (int trial = 0; trial < 60; ++trial) {
        const int B = 1 + trial % 4, H = 1 + trial % 2, D = 16;
        std::vector<int32_t> cq(B + 1, 0), ck(B + 1, 0);
        for (int b = 0; b < B; ++b) {
            cq[b + 1] = cq[b] + (int)(rng() % 40);
            ck[b + 1] = ck[b] + (trial % 3 == 0 ? (int)(rng() % 40) : cq[b + 1] - cq[b]);
        }
        const int Tq = cq[B], Tk = ck[B];
        std::vector<double> q(Tq * H * D), k(Tk * H * D), v(Tk * H * D), dout(Tq * H * D);
        for (double* p : {q.data(), dout.data()})
            for (int i = 0; i < Tq * H * D; ++i) p[i] = nd(rng);
        for (double* p : {k.data(), v.data()})
            for (int i = 0; i < Tk * H * D; ++i) p[i] = nd(rng);
        int64_t left = -1, right = trial % 2 == 0 ? 0 : -1;
        std::vector<int32_t> func;
        int64_t fn = 0, fld = 0;
        if (trial % 5 == 1) {
            left = (int64_t)(rng() % 20);
            right = (int64_t)(rng() % 5) - 1;
        }
        if (trial % 5 == 2 && Tq > 0) {
            fn = 3;
            fld = Tq + 5;
            func.resize(fn * fld);
            for (auto& x : func) x = (int32_t)(rng() % 50) - 5;
        }
        std::vector<double> o(Tq * H * D), dq(Tq * H * D), dk(Tk * H * D), dv(Tk * H * D);
        const int32_t* f = fn ? func.data() : nullptr;
        expect(oracle_hstu_fwd(B, cq.data(), ck.data(), H, D, q.data(), k.data(), v.data(), 0.25, 40.0, left, right, f,
                               fn, fld, nullptr, Tq, o.data()) == 0, "oracle fwd");
        expect(oracle_hstu_bwd_dq(B, cq.data(), ck.data(), H, D, dout.data(), q.data(), k.data(), v.data(), 0.25,
                                  40.0, left, right, f, fn, fld, nullptr, Tq, dq.data()) == 0, "oracle dq");
        expect(oracle_hstu_bwd_dkdv(B, cq.data(), ck.data(), H, D, dout.data(), q.data(), k.data(), v.data(), 0.25,
                                    40.0, left, right, f, fn, fld, nullptr, Tk, dk.data(), dv.data()) == 0,
               "oracle dkdv");
        std::vector<int64_t> rows;
        for (int r = 0; r < Tq; r += 3) rows.push_back(r);
        std::vector<double> o2(rows.size() * H * D);
        expect(oracle_hstu_fwd(B, cq.data(), ck.data(), H, D, q.data(), k.data(), v.data(), 0.25, 40.0, left, right, f,
                               fn, fld, rows.data(), (int64_t)rows.size(), o2.data()) == 0, "oracle fwd rows");
        for (size_t i = 0; i < rows.size(); ++i)
            for (int j = 0; j < H * D; ++j)
                expect(o2[i * H * D + j] == o[rows[i] * H * D + j], "oracle row subset matches");
        for (double x : dq) expect(std::isfinite(x), "oracle dq finite");
    }
    // LMSD with padded strides
    const int n = 37, d = 24, xs = 40, us = 32, s = 3;
    std::vector<double> x(n * xs), u(n * us), w(d), b(d), y(n * s * d), mean(n), rstd(n), dy(n * s * d);
    for (auto& t : x) t = nd(rng);
    for (auto& t : u) t = nd(rng);
    for (auto& t : w) t = 1.0 + 0.1 * nd(rng);
    for (auto& t : b) t = 0.1 * nd(rng);
    for (auto& t : dy) t = nd(rng);
    oracle_lmsd_fwd(n, d, x.data(), xs, u.data(), us, w.data(), b.data(), 1e-6, 1, 1, 1, y.data(), mean.data(),
                    rstd.data());
    std::vector<double> dx(n * d), du(n * d), dw(d), db(d);
    oracle_lmsd_bwd(n, d, dy.data(), s * d, x.data(), xs, u.data(), us, w.data(), b.data(), mean.data(), rstd.data(),
                    1, 1, 1, dx.data(), du.data(), dw.data(), db.data());
    for (double t : dx) expect(std::isfinite(t), "lmsd dx finite");
}

}  // namespace

int main() {
    check_rejections();
    check_oracle();
    if (g_failures) {
        std::fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("abi_check: all checks passed\n");
    return 0;
}
