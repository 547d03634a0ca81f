/* A plain C99 consumer of libhstu's C ABI, built against include/hstu.h alone and
 * linked to libhstu.so.  It runs host-side paths only (no GPU is touched): the
 * version and status strings, workspace-size queries (their values against the
 * sizes the header states), argument rejections with their messages, and the
 * release build's answer to hstu_debug_take.  Prints "ok" and exits 0 when every
 * check holds; otherwise names each failed check and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hstu.h"

static int failures = 0;

static void check(int cond, const char* what) {
    if (!cond) {
        printf("FAILED: %s (last error: %s)\n", what, hstu_last_error());
        ++failures;
    }
}

/* B = 2 causal sequences of up to 32 tokens, H = 2, D = 64, packed strides. */
static hstu_args_t small_args(void) {
    hstu_args_t a;
    memset(&a, 0, sizeof a);
    a.batch = 2;
    a.total_q = 40;
    a.total_k = 40;
    a.num_heads = 2;
    a.head_dim = 64;
    a.max_seqlen_q = 32;
    a.max_seqlen_k = 32;
    a.alpha = 0.125f;
    a.scaling_seqlen = 0;
    a.mask = HSTU_MASK_CAUSAL;
    return a;
}

int main(void) {
    /* a non-null, 256-byte aligned address that is never dereferenced: every call
     * below is refused or answered on the host before any launch */
    void* const fake = (void*)(uintptr_t)0x100000;
    const int32_t* const cu = (const int32_t*)fake;

    check(hstu_abi_version() == HSTU_ABI_VERSION, "ABI version matches the header");
    check(strcmp(hstu_status_string(HSTU_OK), "HSTU_OK") == 0, "status string of HSTU_OK");
    check(strcmp(hstu_status_string(HSTU_ERR_UNSUPPORTED), "HSTU_ERR_UNSUPPORTED") == 0,
          "status string of HSTU_ERR_UNSUPPORTED");

    /* Causal workspace: N = (T_q + 31 B) / 32 = 3 row-block slots, n = 1 row block per
     * longest sequence, k = min(B, N / n) = 2 sequences of n(n + 1)/2 = 1 block, r = 0:
     * 2 blocks of 2 KB per head, H = 2. */
    {
        hstu_args_t a = small_args();
        size_t n = 1;
        check(hstu_bwd_workspace_size(&a, &n) == HSTU_OK, "causal workspace size query");
        check(n == 2u * 2u * 2048u, "causal workspace size is 2 blocks per head");
        a.mask = HSTU_MASK_NONE; /* min(N_q ceil(max_k/32), N_k ceil(max_q/32)) = 3 blocks per head */
        check(hstu_bwd_workspace_size(&a, &n) == HSTU_OK && n == 2u * 3u * 2048u,
              "full-mask workspace size is 3 blocks per head");
        a.total_q = 0; /* no query tokens: nothing to store */
        a.max_seqlen_q = 0;
        check(hstu_bwd_workspace_size(&a, &n) == HSTU_OK && n == 0, "no queries, no workspace");
    }

    /* rejections, each with nothing enqueued */
    {
        hstu_args_t a = small_args();
        a.head_dim = 24;
        check(hstu_fwd(&a, fake, fake, fake, cu, cu, fake, NULL) == HSTU_ERR_UNSUPPORTED, "head_dim 24 refused");
        check(strstr(hstu_last_error(), "head_dim") != NULL, "its message names head_dim");
    }
    {
        hstu_args_t a = small_args();
        a.max_seqlen_q = 33;
        check(hstu_fwd(&a, fake, fake, fake, cu, cu, fake, NULL) == HSTU_ERR_INVALID_ARGUMENT,
              "max_seqlen_q > max_seqlen_k refused");
    }
    {
        hstu_args_t a = small_args();
        check(hstu_fwd(&a, NULL, fake, fake, cu, cu, fake, NULL) == HSTU_ERR_INVALID_ARGUMENT, "null q refused");
        check(hstu_fwd(NULL, fake, fake, fake, cu, cu, fake, NULL) == HSTU_ERR_INVALID_ARGUMENT, "null args refused");
        check(hstu_fwd(&a, fake, fake, fake, NULL, cu, fake, NULL) == HSTU_ERR_INVALID_ARGUMENT,
              "null cu_seqlens_q refused");
    }
    {
        hstu_args_t a = small_args();
        size_t need = 0;
        check(hstu_bwd_workspace_size(&a, &need) == HSTU_OK, "workspace size for the too-small check");
        char* const base = (char*)fake;  /* distinct outputs, each 256-byte aligned */
        check(hstu_bwd(&a, fake, fake, fake, fake, cu, cu, base + 256, base + 512, base + 768, base + 4096,
                       need - 1, NULL) == HSTU_ERR_INVALID_ARGUMENT,
              "a workspace one byte short refused");
        check(strstr(hstu_last_error(), "workspace") != NULL, "its message names the workspace");
    }
    {
        hstu_lmsd_args_t l;
        memset(&l, 0, sizeof l);
        l.n = 4;
        l.d = 64;
        l.eps = 1e-6f;
        l.dropout_ratio = 0.1f;
        check(hstu_lmsd_fwd(&l, fake, fake, fake, fake, fake, (float*)fake, (float*)fake, NULL) ==
                  HSTU_ERR_UNSUPPORTED,
              "LMSD dropout refused");
    }

    /* the release build records no bounds tests */
    {
        uint32_t sites = 7;
        check(hstu_debug_take(NULL) == HSTU_ERR_INVALID_ARGUMENT, "hstu_debug_take(NULL) refused");
        check(hstu_debug_take(&sites) == HSTU_ERR_UNSUPPORTED && sites == 0,
              "hstu_debug_take on the release build: unsupported, 0 written");
    }

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
