/* Exercises the host side of the C ABI in include/mta.h (validation, kernel
 * selection, LDS fit, workspace sizing, argument checks) for an
 * AddressSanitizer / UBSan build of the library's host code
 * (tests/test_sanitize.py).  No call here reaches a kernel launch or any other
 * GPU call: every forward and backward call is given an empty problem, a NULL
 * or a misaligned pointer, or a configuration the checks refuse.  Exit status 0
 * when every call returns what the header documents. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mta.h"

static int fails = 0;
#define EXPECT(cond, ...)                          \
    do {                                           \
        if (!(cond)) {                             \
            fprintf(stderr, __VA_ARGS__);          \
            fputc('\n', stderr);                   \
            ++fails;                               \
        }                                          \
    } while (0)

static float fbuf[4096] __attribute__((aligned(256)));

static mta_config base(void)
{
    mta_config c = {2, 4, 100, 128, 6, 11, 2, MTA_PRE_SOFTMAX, MTA_POST_SOFTMAX, MTA_BF16, 1e-5f, 0.5f};
    return c;
}

static void sweep_configs(void)
{
    const int dts[] = {MTA_F32, MTA_BF16, 2}, ds[] = {16, 32, 64, 128}, chs[] = {1, 2, 3, 4};
    const int Hs[] = {1, 2, 3, 4, 8}, cqs[] = {0, 1, 2, 6, 8, 16, 17}, cks[] = {0, 1, 4, 9, 11, 15, 31, 32};
    long n_ok = 0;
    for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 4; ++b)
            for (int e = 0; e < 4; ++e)
                for (int h = 0; h < 5; ++h)
                    for (int i = 0; i < 7; ++i)
                        for (int j = 0; j < 8; ++j)
                            for (int kq = -1; kq <= 3; ++kq)
                                for (int hp = -1; hp <= 2; ++hp) {
                                    mta_config c = base();
                                    c.dtype = dts[a]; c.head_dim = ds[b]; c.c_h = chs[e]; c.heads = Hs[h];
                                    c.c_q = cqs[i]; c.c_k = cks[j]; c.kq_place = kq; c.head_place = hp;
                                    const int rc = mta_check_config(&c);
                                    const char *name = mta_kernel_name(&c);
                                    EXPECT(rc <= 0 && rc >= MTA_ERR_SCRATCH, "status %d out of range", rc);
                                    EXPECT((rc == MTA_OK) == (name != NULL),
                                           "check_config %d but kernel_name %s", rc, name ? name : "(null)");
                                    if (name) EXPECT(strlen(name) > 8, "short kernel name");
                                    const size_t ws = mta_backward_workspace_size(&c);
                                    const char *bname = mta_backward_kernel_name(&c);
                                    EXPECT((rc == MTA_OK) <= (bname != NULL), "backward name for a valid config");
                                    EXPECT((ws == 0) == (rc != MTA_OK && rc != MTA_ERR_UNSUPPORTED) ||
                                               rc == MTA_ERR_UNSUPPORTED,
                                           "workspace %zu for status %d", ws, rc);
                                    if (rc == MTA_OK) ++n_ok;
                                    /* a misaligned query pointer stops every call before a launch */
                                    const char *q = (const char *)fbuf + 4;
                                    const int fr = mta_forward(q, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, &c, fbuf, NULL);
                                    EXPECT(fr == (rc == MTA_OK ? MTA_ERR_MISALIGNED : fr),
                                           "forward misaligned: %d (config %d)", fr, rc);
                                    const int br = mta_backward(q, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c,
                                                                fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf,
                                                                sizeof fbuf, NULL);
                                    EXPECT(br <= 0, "backward status %d", br);
                                }
    EXPECT(n_ok > 100, "only %ld valid configurations", n_ok);
    printf("config sweep: %ld valid\n", n_ok);
}

static void scalar_checks(void)
{
    mta_config c = base();
    EXPECT(mta_check_config(NULL) == MTA_ERR_NULL_ARG, "NULL config");
    EXPECT(mta_kernel_name(NULL) == NULL, "NULL config name");
    EXPECT(mta_backward_workspace_size(NULL) == 0, "NULL config workspace");
    c.gn_eps = 0.0f;
    EXPECT(mta_check_config(&c) == MTA_ERR_BAD_VALUE, "eps 0");
    c.gn_eps = NAN;
    EXPECT(mta_check_config(&c) == MTA_ERR_BAD_VALUE, "eps NaN");
    c = base();
    c.depth_scale = INFINITY;
    EXPECT(mta_check_config(&c) == MTA_ERR_BAD_VALUE, "depth_scale inf");
    c = base();
    c.batch = -1;
    EXPECT(mta_check_config(&c) == MTA_ERR_BAD_SHAPE, "B < 0");
    c = base();
    c.seq_len = (1 << 24) + 1;
    EXPECT(mta_check_config(&c) == MTA_ERR_UNSUPPORTED, "T > 2^24");
    c = base();
    c.batch = INT32_MAX;
    c.seq_len = 1 << 24;
    EXPECT(mta_check_config(&c) == MTA_ERR_UNSUPPORTED, "grid overflow");
    for (int s = -12; s <= 2; ++s) {
        const char *m = mta_status_string(s);
        EXPECT(m && strlen(m) > 0, "status string %d", s);
    }
    EXPECT(mta_abi_version() > 0, "abi version");

    /* empty problems succeed without touching any pointer */
    c = base();
    c.batch = 0;
    EXPECT(mta_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, &c, NULL, NULL) == MTA_OK, "empty batch");
    c = base();
    c.seq_len = 0;
    EXPECT(mta_forward_gated(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, &c, NULL, NULL) == MTA_OK,
           "empty sequence");
    c = base();
    EXPECT(mta_forward(NULL, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, &c, fbuf, NULL) == MTA_ERR_NULL_ARG, "NULL q");
    EXPECT(mta_forward_gated(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, &c, fbuf, NULL) == MTA_ERR_NULL_ARG,
           "NULL gate");
    EXPECT(mta_forward(fbuf, fbuf, fbuf, (const float *)((const char *)fbuf + 2), fbuf, fbuf, fbuf, &c, fbuf,
                       NULL) == MTA_ERR_MISALIGNED,
           "misaligned theta");

    /* backward argument checks */
    const size_t need = mta_backward_workspace_size(&c);
    EXPECT(need > 0, "workspace size");
    EXPECT(mta_backward(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, &c, fbuf, fbuf, fbuf, fbuf, fbuf,
                        fbuf, fbuf, NULL, fbuf, need, NULL) == MTA_ERR_NULL_ARG,
           "gate without dgate");
    EXPECT(mta_backward(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf, fbuf,
                        fbuf, fbuf, NULL, (char *)fbuf + 16, need, NULL) == MTA_ERR_MISALIGNED,
           "workspace not 256-byte aligned");
    EXPECT(mta_backward(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf, fbuf,
                        fbuf, fbuf, NULL, fbuf, need - 1, NULL) == MTA_ERR_BAD_VALUE,
           "workspace too small");
    /* every placement has a backward; the one with the maps in the workspace
     * takes T <= 32768 and accepts down to one head group's maps */
    c.kq_place = MTA_POST_SOFTMAX;
    c.c_h = 4;
    EXPECT(mta_backward_kernel_name(&c) && strstr(mta_backward_kernel_name(&c), "mta_bwd_gen"),
           "post-softmax backward name");
    EXPECT(mta_backward(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf, fbuf,
                        fbuf, fbuf, NULL, fbuf, 4096, NULL) == MTA_ERR_BAD_VALUE,
           "post-softmax backward, workspace too small");
    c.seq_len = 40000;
    EXPECT(mta_backward_kernel_name(&c) == NULL, "map form beyond T = 32768");
    EXPECT(mta_backward_workspace_size(&c) == 0, "map form workspace beyond T = 32768");
    EXPECT(mta_backward(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf, fbuf,
                        fbuf, fbuf, NULL, fbuf, sizeof fbuf, NULL) == MTA_ERR_UNSUPPORTED,
           "map form beyond T = 32768");
    c = base();
    EXPECT(mta_backward_kernel_name(&c) && strstr(mta_backward_kernel_name(&c), "fused"), "fused backward name");
    /* a problem beyond the device scratch array is refused before any GPU call */
    c = base();
    c.batch = 64;
    c.seq_len = 8192;
    EXPECT(mta_backward_workspace_size(&c) > mta_backward_scratch_bytes(), "scratch sizing");
    EXPECT(mta_backward_noalloc(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf,
                                fbuf, fbuf, fbuf, NULL, NULL) == MTA_ERR_SCRATCH,
           "noalloc refusal");
    c.c_h = 3;
    EXPECT(mta_backward_noalloc(fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, fbuf, NULL, fbuf, &c, fbuf, fbuf, fbuf, fbuf,
                                fbuf, fbuf, fbuf, NULL, NULL) == MTA_ERR_BAD_SHAPE,
           "noalloc validation");
}

static void layer_sweep(void)
{
    long n_ok = 0, n_rep = 0;
    for (int dt = 0; dt < 2; ++dt)
        for (int ch = 1; ch <= 4; ch *= 2)
            for (int exact = 0; exact <= 1; ++exact)
                for (int mask = 0; mask < 64; ++mask)
                    for (int ks = 0; ks < 6; ++ks) {
                        /* ks >= 3: head_dim 128 with the same kernel size after the
                           softmax (the repeated form's head-split kernel at 6x11, 4x9, 1x1) */
                        const int cq[] = {6, 16, 1, 6, 4, 1}, ck[] = {11, 31, 1, 11, 9, 1};
                        const int d = ks < 3 ? 64 : 128, cq2 = ks < 3 ? 2 : cq[ks], ck2 = ks < 3 ? 3 : ck[ks];
                        mta_layer_config c = {2, 4, 77, d, cq[ks], ck[ks], cq2, ck2, ch, exact, dt, 1e-5f, 1.0f};
                        mta_layer_weights w;
                        memset(&w, 0, sizeof w);
                        w.kq_pre = (mask & 1) ? fbuf : NULL;
                        w.head_pre = (mask & 2) ? fbuf : NULL;
                        w.conv3d = (mask & 4) ? fbuf : NULL;
                        w.head_post = (mask & 8) ? fbuf : NULL;
                        w.kq_post = (mask & 16) ? fbuf : NULL;
                        w.head_post2 = (mask & 32) ? fbuf : NULL;
                        w.gn_w = fbuf;
                        w.gn_b = fbuf;
                        const char *name = mta_layer_kernel_name(&c, &w);
                        if (name) {
                            EXPECT(strlen(name) > 8, "short layer kernel name");
                            ++n_ok;
                            if (strncmp(name, "mta_fwd_rep", 11) == 0) {
                                ++n_rep;
                                EXPECT(dt == MTA_BF16 && d == 128 && ch == 2 && !exact && w.kq_pre && w.kq_post &&
                                           !w.head_pre && !w.conv3d,
                                       "repeated-form kernel chosen outside its scope");
                            }
                        }
                        const int rc = mta_forward_layer((const char *)fbuf + 4, fbuf, fbuf, &w, &c, fbuf, NULL);
                        EXPECT(rc < 0, "layer forward with a misaligned q returned %d", rc);
                        EXPECT(mta_forward_layer(NULL, fbuf, fbuf, &w, &c, fbuf, NULL) < 0, "layer NULL q");
                        c.batch = 0;
                        EXPECT(mta_forward_layer(NULL, NULL, NULL, &w, &c, NULL, NULL) <= 0, "layer empty");
                    }
    EXPECT(mta_layer_kernel_name(NULL, NULL) == NULL, "layer NULL");
    EXPECT(n_ok > 50, "only %ld layer forms accepted", n_ok);
    EXPECT(n_rep == 12, "the repeated-form kernel chosen %ld times (expected 12)", n_rep);
    printf("layer sweep: %ld accepted, %ld on the repeated form's kernel\n", n_ok, n_rep);
}

int main(void)
{
    scalar_checks();
    sweep_configs();
    layer_sweep();
    if (fails) {
        fprintf(stderr, "%d failed checks\n", fails);
        return 1;
    }
    printf("abi driver: ok\n");
    return 0;
}
