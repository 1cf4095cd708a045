/* A plain C99 caller of libla.so: the header compiles as C and the exported
 * entry points link and answer. Only calls that need no GPU are made: the
 * queries, and calls that fail argument validation before any HIP call. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "la.h"

static int fails = 0;
#define CHECK(cond)                                            \
    do {                                                       \
        if (!(cond)) {                                         \
            fprintf(stderr, "check failed: %s\n", #cond);      \
            ++fails;                                           \
        }                                                      \
    } while (0)

int main(void) {
    la_problem p;
    memset(&p, 0, sizeof p); /* zero-initialised: Dv = D, scale = 1 */
    p.B = 2;
    p.H = 3;
    p.T = 100;
    p.D = 64;
    p.dtype = LA_F16;
    p.eps = 1e-6f;

    CHECK(la_version() == LA_VERSION);
    CHECK(strncmp(la_status_str(LA_ERR_HEAD_DIM), "LA_ERR_HEAD_DIM", 15) == 0);
    CHECK(la_state_bytes(&p) == (size_t)(2 * 3 * (64 * 64 + 64) * 4));
    CHECK(la_workspace_bytes(&p) > 0);
    {
        la_split sp;
        CHECK(la_split_of(&p, &sp) == LA_OK);
        CHECK(sp.P >= 1 && sp.P * sp.L >= p.T && sp.NK >= 1 && sp.NK * sp.LK >= p.T);
        CHECK(la_split_of(&p, NULL) == LA_ERR_NULL);
    }

    /* validation errors, before any HIP call */
    CHECK(la_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_NULL);
    CHECK(la_fwd_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, NULL) == LA_ERR_NULL);
    CHECK(LA_NOALLOC_SCRATCH_BYTES == 64u * 1024u * 1024u);
    p.D = 48;
    CHECK(la_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_HEAD_DIM);
    p.D = 64;
    p.eps = -1.0f;
    CHECK(la_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_EPS);
    p.eps = 1e-6f;
    p.scale = NAN;
    CHECK(la_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_SCALE);
    p.scale = 0.0f;
    p.flags = LA_CAUSAL;
    CHECK(la_fwd_state(&p, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_FLAGS);
    p.dtype = LA_F32; /* the causal form takes fp32 too: the missing workspace is reported */
    CHECK(la_bwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_WORKSPACE);
    p.D = 256;
    p.dtype = LA_F16;
    CHECK(la_bwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_HEAD_DIM);
    p.D = 64;
    /* reusing the forward's prefixes: causal la_fwd / la_bwd only */
    p.flags = LA_CAUSAL | LA_REUSE_PREFIX;
    CHECK(la_bwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_WORKSPACE);
    CHECK(la_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_WORKSPACE);
    CHECK(la_fwd_noalloc(&p, NULL, NULL, NULL, NULL, NULL, NULL) == LA_ERR_FLAGS);
    p.flags = LA_REUSE_PREFIX;
    CHECK(la_bwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LA_ERR_FLAGS);

    if (fails == 0) printf("c abi ok\n");
    return fails == 0 ? 0 : 1;
}
