/* Test support: drives the C ABI's host code (built with the launch stubs
 * and the host sanitizers) through its validation paths and through a
 * launch that fails, checking every status code; prints "ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/sharq.h"

static int fails = 0;
#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        int got_ = (int)(call);                                                                     \
        if (got_ != (want)) {                                                                       \
            printf("line %d: %s gave %d, expected %d\n", __LINE__, #call, got_, (int)(want));       \
            fails++;                                                                                \
        }                                                                                           \
    } while (0)

int main(void) {
    /* aligned and misaligned stand-ins for device pointers: never dereferenced */
    void *P = (void *)(uintptr_t)0x10000, *MIS = (void *)(uintptr_t)0x10002;
    uint8_t *U = (uint8_t *)P;
    float *F = (float *)P;
    const int BF = SHARQ_BF16, MX = SHARQ_MXFP4, NV = SHARQ_NVFP4, SP = SHARQ_NVFP4_SP24;

    EXPECT(sharq_abi_version(), SHARQ_ABI_VERSION);
    for (int s = 0; s < 10; s++)
        if (!sharq_status_string(s)) fails++;
    EXPECT(sharq_last_hip_error(), 0);

    /* sharq_prepare: every validation status, then a launch that fails */
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, 7, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_UNSUPPORTED);
    EXPECT(sharq_prepare(P, SHARQ_F32, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_DTYPE);
    EXPECT(sharq_prepare(P, BF, 4, 100, 100, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare(P, BF, -1, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare(P, BF, INT64_MAX, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 5, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_NM);
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 3, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_NM);
    EXPECT(sharq_prepare(NULL, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_NULL);
    EXPECT(sharq_prepare(MIS, BF, 4, 256, 256, 0, NULL, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_ALIGN);
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, NV, U, U, U, U, U, F, NULL, 0, NULL),
           SHARQ_ERR_WORKSPACE);
    EXPECT(sharq_prepare(NULL, BF, 0, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_OK);
    EXPECT(sharq_last_hip_error(), 0);
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_HIP);
    EXPECT(sharq_last_hip_error(), 1 /* hipErrorInvalidValue */);
    EXPECT(sharq_prepare_noalloc(P, BF, SHARQ_NOALLOC_MAX_ROWS + 1, 256, 256, 1, P, NULL, 1e-5f, 2, 4, NV, U, U, U,
                                 U, U, F, NULL),
           SHARQ_ERR_WORKSPACE);
    EXPECT(sharq_prepare_noalloc(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, MX, U, U, U, U, U, NULL, NULL),
           SHARQ_ERR_HIP);

    /* NVFP4_SP24: the 2:4 mask, whole K tiles, 32-bit code offsets */
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 4, 8, SP, U, U, U, U, U, F, NULL, 0, NULL),
           SHARQ_ERR_NM);
    EXPECT(sharq_prepare(P, BF, 4, 160, 160, 1, P, NULL, 1e-5f, 2, 4, SP, U, U, U, U, U, F, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare(P, BF, (int64_t)1 << 24, 512, 512, 1, P, NULL, 1e-5f, 2, 4, SP, U, U, U, U, U, F, NULL, 0,
                         NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare(P, BF, 4, 256, 256, 1, P, NULL, 1e-5f, 2, 4, SP, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_NULL);
    EXPECT(sharq_prepare_swiglu(F, 4, 160, 320, 2, 4, SP, U, U, U, U, U, F, NULL, 0, NULL), SHARQ_ERR_SHAPE);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, SP, U, U, F, 1, 64, NULL, NULL, 4, P, SHARQ_F32, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_NULL);
    EXPECT(sharq_linear(U, U, U, U, F, 4, 256, SP, U, U, F, 1, 64, NULL, NULL, 4, P, SHARQ_F32, 64, NULL, 0, NULL),
           SHARQ_ERR_HIP);

    /* sharq_prepare_swiglu */
    EXPECT(sharq_prepare_swiglu(F, 4, 256, 300, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_SHAPE);
    EXPECT(sharq_prepare_swiglu((const float *)MIS, 4, 256, 512, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL),
           SHARQ_ERR_ALIGN);
    EXPECT(sharq_prepare_swiglu(F, 4, 256, 512, 2, 4, MX, U, U, U, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_HIP);

    /* sharq_quantize_weight */
    EXPECT(sharq_quantize_weight(P, BF, 1, 16, 256, 128, MX, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_SHAPE);
    EXPECT(sharq_quantize_weight(P, BF, 1, 16, 256, 256, NV, U, U, F, NULL, 0, NULL), SHARQ_ERR_WORKSPACE);
    EXPECT(sharq_quantize_weight(P, BF, 1, 16, 256, 256, MX, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_HIP);

    /* sharq_linear */
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, MX, U, U, NULL, 1, 64, NULL, NULL, 4, P, 9, 64, NULL, 0, NULL),
           SHARQ_ERR_DTYPE);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 160, MX, U, U, NULL, 1, 64, NULL, NULL, 4, P, SHARQ_F32, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, MX, U, U, NULL, 4, 64, NULL, NULL, 4, P, SHARQ_F32, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_NULL);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, MX, U, U, NULL, 1, 64, NULL, NULL, 4, MIS, SHARQ_F32, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_ALIGN);
    EXPECT(sharq_linear(U, U, U, U, NULL, ((int64_t)1 << 40), 256, MX, U, U, NULL, 1, 64, NULL, NULL,
                        ((int64_t)1 << 40), P, SHARQ_F32, 64, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, MX, U, U, NULL, 1, 64, NULL, NULL, 4, P, SHARQ_BF16, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_HIP);

    /* sharq_quantize_weight_gate_up, sharq_linear_swiglu */
    EXPECT(sharq_quantize_weight_gate_up(P, BF, 1, 96, 256, 256, MX, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_SHAPE);
    EXPECT(sharq_quantize_weight_gate_up(P, BF, 1, 128, 256, 256, MX, U, U, NULL, NULL, 0, NULL), SHARQ_ERR_HIP);
    EXPECT(sharq_linear_swiglu(U, U, U, U, 4, 256, U, U, 1, 320, NULL, NULL, 4, 2, 4, U, U, U, U, U, NULL, 0, NULL),
           SHARQ_ERR_SHAPE);
    EXPECT(sharq_linear_swiglu(U, U, U, U, 4, 256, U, U, 1, 512, NULL, NULL, 4, 2, 8, U, U, U, U, U, NULL, 0, NULL),
           SHARQ_ERR_UNSUPPORTED);
    EXPECT(sharq_linear_swiglu(U, U, U, U, 4, 256, U, U, 1, 512, NULL, NULL, 4, 2, 4, U, MIS, U, U, U, NULL, 0,
                               NULL),
           SHARQ_ERR_ALIGN);
    EXPECT(sharq_linear_swiglu(U, U, U, U, 4, 256, U, U, 1, 512, NULL, NULL, 4, 2, 4, U, U, U, U, U, F, 512, NULL),
           SHARQ_ERR_HIP);

    /* check mode: the failed launch is reported the same way */
    setenv("SHARQ_DEBUG", "1", 1);
    EXPECT(sharq_linear(U, U, U, U, NULL, 4, 256, MX, U, U, NULL, 1, 64, NULL, NULL, 4, P, SHARQ_F32, 64, NULL, 0,
                        NULL),
           SHARQ_ERR_HIP);
    EXPECT(sharq_last_hip_error(), 1);

    if (fails == 0) printf("ok\n");
    return fails == 0 ? 0 : 1;
}
