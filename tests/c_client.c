/* A plain C client of libspecconv: include/specconv.h compiles as C99 and the library
 * links and answers host-side queries.  Only calls that return before any HIP work are made
 * (argument checks, sizes, strings), so this runs without a GPU. */
#include "specconv.h"

#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main(void)
{
    CHECK(sc_version() >= 800);
    CHECK(strcmp(sc_status_string(SC_OK), "SC_OK") == 0);
    /* negative sizes and null pointers with work to do are rejected on the host */
    CHECK(sc_causal_conv_f32(0, 0, 0, -1, 1, 1, 0) == SC_ERR_INVALID_ARGUMENT);
    CHECK(sc_causal_conv_bf16(0, 0, 0, 1, 1, 1, 0) == SC_ERR_INVALID_ARGUMENT);
    /* lengths beyond a kind's path (placeholder pointers, never dereferenced) */
    CHECK(sc_causal_conv_ntt_i32((const int32_t*)0x100000, (const int32_t*)0x200000,
                                 (int32_t*)0x300000, 1, 1, 65537, 0) == SC_ERR_UNSUPPORTED);
    /* empty calls are no-ops */
    CHECK(sc_causal_conv_f32(0, 0, 0, 0, 4, 64, 0) == SC_OK);
    /* sizes */
    CHECK(sc_workspace_bytes(SC_KIND_F32, 8, 1024, 4096) == 0);          /* fused path */
    CHECK(sc_workspace_bytes(SC_KIND_F32, 1, 1536, 65536) > 0);          /* four-step */
    CHECK(sc_filter_spectrum_bytes(3, 100) == (size_t)3 * (2 * 128 + 32) * 8);
    CHECK(sc_blc_workspace_bytes(SC_KIND_F32, 1, 256, 64) == (size_t)3 * 64 * 1024);
    CHECK(sc_ntt_range_ok(127, 127, 4096) == 1);
    CHECK(sc_ntt_range_ok(1 << 20, 1 << 20, 4096) == 0);
    /* options through the _ex call: an unknown path is an invalid argument */
    {
        sc_options o;
        memset(&o, 0, sizeof o);
        o.path = 9;
        o.head = -1;
        CHECK(sc_causal_conv_ex(SC_KIND_F32, (const void*)0x100000, (const void*)0x200000,
                                (void*)0x300000, 1, 1, 64, &o, 0, 0, 0) ==
              SC_ERR_INVALID_ARGUMENT);
    }
    if (fails) return 1;
    printf("c client ok\n");
    return 0;
}
