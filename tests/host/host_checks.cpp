// Host-side checks of libdc1d's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's host code and on this driver
// (tests/test_host_sanitizers.py builds and runs it; no GPU is used).  Every
// call below is malformed and must be rejected with the documented status
// before any device work; the sanitizers watch the validation code for
// out-of-bounds accesses, overflowing arithmetic on the shapes and other
// undefined behaviour.  Data pointers are fake: validation never
// dereferences them, and no call here reaches a launch.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "dc1d.h"

static int failures = 0;

#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const int got_ = (int)(call);                                                               \
        if (got_ != (int)(want)) {                                                                  \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
                    (int)(want));                                                                   \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

static void *const FAKE = (void *)(uintptr_t)0x10000000;

static dc1d_tensor T(int dtype, int ndim, int64_t s0, int64_t s1 = 0, int64_t s2 = 0, int64_t s3 = 0,
                     uintptr_t addr = 0x10000000) {
    dc1d_tensor t;
    t.data = (void *)addr;
    t.dtype = dtype;
    t.ndim = ndim;
    t.shape[0] = s0;
    t.shape[1] = s1;
    t.shape[2] = s2;
    t.shape[3] = s3;
    return t;
}

int main() {
    const int64_t BIG = (int64_t)1 << 62, HUGE = INT64_MAX;
    const uintptr_t step = (uintptr_t)1 << 24;
    // ---- output length
    EXPECT(dc1d_output_length(HUGE, 3, 1, 0, 1), -1);
    EXPECT(dc1d_output_length(10, HUGE, 1, 0, 1), -1);
    EXPECT(dc1d_output_length(10, 3, 1, HUGE, 1), -1);
    EXPECT(dc1d_output_length(10, 3, 1, 0, HUGE), -1);
    EXPECT(dc1d_output_length(10, 3, HUGE, 0, 1), 1);
    EXPECT(dc1d_output_length(-5, 3, 1, 0, 1), -1);
    EXPECT(dc1d_output_length(128, 16, 1, 0, 3), 83);

    // ---- forward: a valid layout to break one argument at a time
    dc1d_tensor x = T(DC1D_F32, 3, 2, 8, 20, 0, 0x10000000);
    dc1d_tensor off = T(DC1D_F32, 4, 2, 2, 18, 3, 0x10000000 + step);
    dc1d_tensor mask = T(DC1D_F32, 4, 2, 2, 18, 3, 0x10000000 + 2 * step);
    dc1d_tensor w = T(DC1D_F32, 3, 6, 8, 3, 0, 0x10000000 + 3 * step);
    dc1d_tensor bias = T(DC1D_F32, 1, 6, 0, 0, 0, 0x10000000 + 4 * step);
    dc1d_tensor out = T(DC1D_F32, 3, 2, 6, 18, 0, 0x10000000 + 5 * step);
    EXPECT(dc1d_forward(nullptr, &off, &mask, &w, &bias, &out, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_NULL_PTR);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, nullptr, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_NULL_PTR);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, &out, 0, 0, 1, 1, 2, nullptr, 0, nullptr), DC1D_ERR_BAD_ARG);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, &out, 1, -1, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_ARG);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, &out, 1, 0, 1, 1, 4, nullptr, 0, nullptr), DC1D_ERR_BAD_ARG);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, &out, HUGE, HUGE, HUGE, HUGE, HUGE, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);  // sizes beyond the supported limits
    // shapes near the int64 range: rejected without overflowing arithmetic
    dc1d_tensor xb = T(DC1D_F32, 3, BIG, BIG, BIG);
    dc1d_tensor wb = T(DC1D_F32, 3, BIG, BIG, BIG, 0, 0x10000000 + 3 * step);
    EXPECT(dc1d_forward(&xb, &off, nullptr, &w, nullptr, &out, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    EXPECT(dc1d_forward(&x, &off, nullptr, &wb, nullptr, &out, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor xh = T(DC1D_F32, 3, HUGE, HUGE, HUGE);
    dc1d_tensor wh = T(DC1D_F32, 3, HUGE, HUGE, HUGE, 0, 0x10000000 + 3 * step);
    EXPECT(dc1d_forward(&xh, &off, nullptr, &wh, nullptr, &out, 1, 0, 1, 1, 1, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    size_t nbytes = 0;
    EXPECT(dc1d_workspace_bytes(&xh, &off, nullptr, &wh, nullptr, 1, 0, 1, 1, 1, &nbytes), DC1D_ERR_BAD_SHAPE);
    EXPECT(dc1d_workspace_bytes(&x, &off, &mask, &w, &bias, 1, 0, 1, 1, 2, nullptr), DC1D_ERR_NULL_PTR);
    // dtypes, ranks, empty sequence, aliasing
    dc1d_tensor x7 = T(7, 3, 2, 8, 20);
    EXPECT(dc1d_forward(&x7, &off, &mask, &w, &bias, &out, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_DTYPE);
    dc1d_tensor x2 = T(DC1D_F32, 2, 2, 8);
    EXPECT(dc1d_forward(&x2, &off, &mask, &w, &bias, &out, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor x0 = T(DC1D_F32, 3, 2, 8, 0, 0, 0);
    dc1d_tensor off0 = T(DC1D_F32, 4, 2, 2, 2, 3, 0x10000000 + step);
    dc1d_tensor out0 = T(DC1D_F32, 3, 2, 6, 2, 0, 0x10000000 + 5 * step);
    EXPECT(dc1d_forward(&x0, &off0, nullptr, &w, nullptr, &out0, 1, 2, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor out_on_x = T(DC1D_F32, 3, 2, 6, 18, 0, 0x10000000 + 64);
    EXPECT(dc1d_forward(&x, &off, &mask, &w, &bias, &out_on_x, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_ALIAS);
    EXPECT(dc1d_forward_constrained(&x, &off, &mask, &w, &bias, &out_on_x, 1, 0, 1, 1, 2, nullptr, 0, nullptr),
           DC1D_ERR_ALIAS);
    EXPECT(dc1d_forward_noalloc(&x, &off, &mask, &w, &bias, nullptr, 1, 0, 1, 1, 2, nullptr), DC1D_ERR_NULL_PTR);
    EXPECT(dc1d_forward_noalloc(&xh, &off, nullptr, &wh, nullptr, &out, 1, 0, 1, 1, 1, nullptr),
           DC1D_ERR_BAD_SHAPE);

    // ---- positions entry
    int32_t *i0 = (int32_t *)FAKE;
    EXPECT(dc1d_debug_positions(nullptr, 20, 1, 0, 1, i0, (float *)FAKE, (uint8_t *)FAKE, nullptr),
           DC1D_ERR_NULL_PTR);
    dc1d_tensor offh = T(DC1D_F32, 4, BIG, BIG, 18, 3);
    EXPECT(dc1d_debug_positions(&offh, 20, 1, 0, 1, i0, (float *)FAKE, (uint8_t *)FAKE, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor offk = T(DC1D_F32, 4, 1, 1, 18, HUGE);
    EXPECT(dc1d_debug_positions(&offk, 20, 1, 0, 1, i0, (float *)FAKE, (uint8_t *)FAKE, nullptr),
           DC1D_ERR_BAD_SHAPE);

    // ---- backward
    dc1d_tensor gx = T(DC1D_F32, 3, 2, 8, 20, 0, 0x10000000 + 8 * step);
    EXPECT(dc1d_backward(&x, &off, &mask, &w, nullptr, &gx, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1, 2,
                         nullptr, 0, nullptr),
           DC1D_ERR_NULL_PTR);
    dc1d_tensor gx_bad = T(DC1D_F32, 3, 2, 8, 19, 0, 0x10000000 + 8 * step);
    EXPECT(dc1d_backward(&x, &off, &mask, &w, &out, &gx_bad, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1, 2,
                         nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor gx_on_x = T(DC1D_F32, 3, 2, 8, 20, 0, 0x10000000 + 16);
    EXPECT(dc1d_backward(&x, &off, &mask, &w, &out, &gx_on_x, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1, 2,
                         nullptr, 0, nullptr),
           DC1D_ERR_ALIAS);
    EXPECT(dc1d_backward(&xh, &off, nullptr, &wh, &out, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1, 1,
                         nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    EXPECT(dc1d_backward_workspace_bytes(&x, &off, &mask, &w, &out, 1, 1, 0, 1, 1, 2, nullptr), DC1D_ERR_NULL_PTR);

    // ---- packed layer
    dc1d_tensor tw = T(DC1D_F32, 3, 8, 1, 3, 0, 0x10000000 + 9 * step);
    dc1d_tensor ow = T(DC1D_F32, 3, 6, 8, 1, 0, 0x10000000 + 10 * step);
    dc1d_tensor owh = T(DC1D_F32, 3, BIG, BIG, 1, 0, 0x10000000 + 10 * step);
    EXPECT(dc1d_packed_workspace_bytes(&x, &tw, &owh, nullptr, &w, 1, 0, 1, 1, &nbytes), DC1D_ERR_BAD_SHAPE);
    EXPECT(dc1d_packed_workspace_bytes(&xh, &tw, &ow, nullptr, &w, 1, 0, 1, 1, &nbytes), DC1D_ERR_BAD_SHAPE);
    EXPECT(dc1d_packed_forward(&x, &tw, nullptr, &ow, nullptr, nullptr, nullptr, &w, nullptr, nullptr, nullptr,
                               nullptr, 1, 0, 1, 1, nullptr, 0, nullptr),
           DC1D_ERR_NULL_PTR);

    // ---- 2D
    dc1d_tensor x4 = T(DC1D_F32, 4, 1, 4, 5, 5);
    dc1d_tensor w4 = T(DC1D_F32, 4, 6, 4, 3, 3, 0x10000000 + 3 * step);
    dc1d_tensor o4 = T(DC1D_F32, 4, 1, 18, 3, 3, 0x10000000 + step);
    dc1d_tensor out4 = T(DC1D_F32, 4, 1, 6, 3, 3, 0x10000000 + 5 * step);
    dc1d_tensor x4h = T(DC1D_F32, 4, BIG, BIG, BIG, BIG);
    EXPECT(dc2d_forward(&x4h, &o4, nullptr, &w4, nullptr, &out4, 1, 1, 0, 0, 1, 1, 1, 1, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    dc1d_tensor w4h = T(DC1D_F32, 4, 6, 4, HUGE, HUGE, 0x10000000 + 3 * step);
    EXPECT(dc2d_forward(&x4, &o4, nullptr, &w4h, nullptr, &out4, 1, 1, 0, 0, 1, 1, 1, 1, nullptr, 0, nullptr),
           DC1D_ERR_BAD_SHAPE);
    EXPECT(dc2d_forward(&x4, &o4, nullptr, &w4, nullptr, &out4, 1, 1, 0, 0, 1, 1, 1, 3, nullptr, 0, nullptr),
           DC1D_ERR_BAD_ARG);
    EXPECT(dc2d_workspace_bytes(&x4, &o4, nullptr, &w4, nullptr, 1, 1, 0, 0, 1, 1, 1, 1, nullptr),
           DC1D_ERR_NULL_PTR);

    // ---- misc
    for (int st = -3; st < 12; ++st)
        if (!dc1d_status_string(st)[0]) ++failures;
    EXPECT(dc1d_set_kernel_events(nullptr, FAKE), DC1D_ERR_NULL_PTR);
    EXPECT(dc1d_set_kernel_events(nullptr, nullptr), DC1D_OK);
    if (dc1d_noalloc_scratch_bytes() != ((size_t)64 << 20)) ++failures;

    printf("host checks: %d failure(s)\n", failures);
    return failures ? 1 : 0;
}
