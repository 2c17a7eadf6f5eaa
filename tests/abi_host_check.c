/* Host-side checks of libmoe's C ABI without a GPU, built and run under
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_host_sanitizers.py
 * (the library's host code compiled with the same sanitizers).
 *
 * Every call below is decided on the host: size and capacity queries, and
 * argument validation that must fail before anything is enqueued.  The
 * program prints one line per failed expectation and exits non-zero if
 * there was any. */
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>

#include "moe.h"

static int failures = 0;

#define EXPECT(cond, what)                                       \
    do {                                                         \
        if (!(cond)) {                                           \
            printf("FAILED: %s (line %d)\n", what, __LINE__);    \
            ++failures;                                          \
        }                                                        \
    } while (0)

static moe_config cfg(int S, int d, int h, int E, int k, double cf, int cap, int bf16,
                      uint32_t flags) {
    moe_config c;
    c.S = S;
    c.d_model = d;
    c.d_ff = h;
    c.E = E;
    c.k = k;
    c.capacity_factor = cf;
    c.capacity = cap;
    c.act_dtype = bf16 ? MOE_BF16 : MOE_F32;
    c.flags = flags;
    return c;
}

int main(void) {
    /* the layer shapes of the benchmark, in every routing mode */
    const int shapes[5][5] = {{256, 64, 128, 8, 2},
                              {16384, 1024, 4096, 128, 2},
                              {16384, 1024, 4096, 128, 2},
                              {65536, 2048, 8192, 64, 2},
                              {8192, 7168, 2048, 256, 8}};
    const double cfs[5] = {1.25, 2.0, 1.0, 1.25, 1.5};
    const int want_c[5] = {80, 512, 256, 2560, 384};
    const uint32_t modes[3] = {0u, MOE_CFG_DROPLESS, MOE_CFG_REROUTE};
    for (int i = 0; i < 5; ++i) {
        for (int m = 0; m < 3; ++m) {
            const int bf16 = i > 0;
            moe_config c = cfg(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3],
                               shapes[i][4], cfs[i], 0, bf16, modes[m]);
            const int32_t C = moe_capacity(&c);
            EXPECT(C == (modes[m] == MOE_CFG_DROPLESS ? shapes[i][0] : want_c[i]), "capacity");
            const int64_t rows = moe_dispatch_rows(&c);
            EXPECT(rows == (modes[m] == MOE_CFG_DROPLESS ? (int64_t)shapes[i][0] * shapes[i][4]
                                                          : (int64_t)shapes[i][3] * C),
                   "dispatch rows");
            size_t ws = 0, bws = 0;
            EXPECT(moe_workspace_bytes(&c, &ws) == MOE_OK && ws > 0, "workspace bytes");
            const moe_status bs = moe_backward_workspace_bytes(&c, &bws);
            EXPECT(bf16 ? (bs == MOE_OK && bws > 0) : bs == MOE_ERR_UNSUPPORTED,
                   "backward workspace bytes");
        }
    }

    /* invalid configurations */
    moe_config bad[8];
    bad[0] = cfg(-1, 64, 64, 8, 2, 1.0, 0, 1, 0);
    bad[1] = cfg(10, 0, 64, 8, 2, 1.0, 0, 1, 0);
    bad[2] = cfg(10, 64, 64, 0, 1, 1.0, 0, 1, 0);
    bad[3] = cfg(10, 64, 64, 4, 5, 1.0, 0, 1, 0);
    bad[4] = cfg(10, 64, 64, 4, 2, 0.0, 0, 1, 0);
    bad[5] = cfg(10, 64, 64, 4, 2, 1.0, -3, 1, 0);
    bad[6] = cfg(10, 64, 64, 4, 2, 1.0, 0, 1, 4u);
    bad[7] = cfg(10, 64, 64, 4, 2, 1.0, 0, 1, MOE_CFG_DROPLESS | MOE_CFG_REROUTE);
    for (int i = 0; i < 8; ++i) {
        size_t n = 0;
        EXPECT(moe_workspace_bytes(&bad[i], &n) == MOE_ERR_INVALID_ARG, "invalid config");
        EXPECT(moe_capacity(&bad[i]) == -1, "invalid config capacity");
        EXPECT(moe_dispatch_rows(&bad[i]) == -1, "invalid config rows");
    }
    EXPECT(moe_workspace_bytes(NULL, NULL) == MOE_ERR_INVALID_ARG, "null config");

    /* entry points with invalid arguments: rejected before any launch.  The
     * fake pointer is never dereferenced. */
    moe_config c = cfg(1000, 256, 512, 16, 2, 1.0, 0, 1, 0);
    size_t ws = 0;
    EXPECT(moe_workspace_bytes(&c, &ws) == MOE_OK, "workspace");
    void* fake = (void*)(uintptr_t)(1u << 20);
    void* odd = (void*)(uintptr_t)((1u << 20) + 4);
    float* ff = (float*)fake;
    int32_t* fi = (int32_t*)fake;
    EXPECT(moe_gate(&c, NULL, ff, NULL, ff, fi, ff, fi, fi, ff, 0u, fake, ws, NULL) ==
               MOE_ERR_INVALID_ARG,
           "gate without x");
    EXPECT(moe_gate(&c, odd, ff, NULL, ff, fi, ff, fi, fi, ff, 0u, fake, ws, NULL) ==
               MOE_ERR_INVALID_ARG,
           "gate with misaligned x");
    EXPECT(moe_gate(&c, fake, ff, NULL, ff, fi, ff, fi, fi, ff, 0u, fake, 256, NULL) ==
               MOE_ERR_WORKSPACE,
           "gate with a small workspace");
    EXPECT(moe_gate(&c, fake, (const float*)odd, NULL, ff, fi, ff, fi, fi, ff, 0u, fake, ws,
                    NULL) == MOE_ERR_INVALID_ARG,
           "gate with misaligned w_gate");
    EXPECT(moe_dispatch(&c, fake, fi, fi, odd, NULL) == MOE_ERR_INVALID_ARG,
           "dispatch with misaligned xd");
    EXPECT(moe_combine(&c, fake, fi, fi, ff, odd, NULL) == MOE_ERR_INVALID_ARG,
           "combine with misaligned y");
    EXPECT(moe_expert_ffn(&c, fake, fi, fake, NULL, fake, NULL, fake, fake, ws / 2, NULL) ==
               MOE_ERR_WORKSPACE,
           "expert ffn with a small workspace");
    EXPECT(moe_layer_forward(&c, fake, ff, NULL, fake, NULL, NULL, NULL, fake, ff, fi, ff, fi,
                             fi, ff, NULL, NULL, NULL, fake, ws, NULL, NULL) ==
               MOE_ERR_INVALID_ARG,
           "forward without w2");
    size_t bws = 0;
    EXPECT(moe_backward_workspace_bytes(&c, &bws) == MOE_OK, "backward workspace");
    EXPECT(moe_layer_backward(&c, fake, ff, fake, NULL, fake, ff, fi, ff, fi, fi, fake, NULL,
                              fake, 0.f, 0.f, fake, (float*)odd, NULL, fake, NULL, fake, NULL,
                              fake, bws, NULL, NULL) == MOE_ERR_INVALID_ARG,
           "backward with misaligned dw_gate");
    EXPECT(moe_layer_backward(&c, fake, ff, fake, NULL, fake, ff, fi, ff, fi, fi, fake, NULL,
                              NULL, 0.f, 0.f, fake, ff, NULL, fake, NULL, fake, NULL, fake, bws,
                              NULL, NULL) == MOE_ERR_INVALID_ARG,
           "backward without dy");
    for (int s = 0; s <= 4; ++s)
        EXPECT(moe_status_string(s) != NULL, "status string");

    printf("%s: %d failed expectations\n", failures ? "FAIL" : "ok", failures);
    return failures ? 1 : 0;
}
