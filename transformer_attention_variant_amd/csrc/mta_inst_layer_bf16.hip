// General-layer kernels, bfloat16 (d in {32, 64, 128}, c_h in {1, 2, 4}).
#include "mta_fwd_layer.h"

namespace mta {

// cq1/ck1: pre-softmax kernel size (0 without one); cq2/ck2: post-softmax one.
layer::LayerFn find_launch_layer_bf16(int d, int ch, int cq1, int ck1, int cq2, int ck2)
{
    // compile-time stencils for the 4K-context layer's forms (6x11, c_h = 2):
    // the repeated convolution (6x11 after the softmax too) and the 3D kernel
    if (d == 128 && ch == 2 && cq1 == 6 && ck1 == 11) {
        if (cq2 == 6 && ck2 == 11) return &layer::launch<bf16_t, 128, 2, 6, 11, 6, 11>;
        if (cq2 == 0) return &layer::launch<bf16_t, 128, 2, 6, 11, 0, 0>;
    }
#define MTA_LAYER_CH(D_)                                        \
    switch (ch) {                                               \
    case 1: return &layer::launch<bf16_t, D_, 1>;                \
    case 2: return &layer::launch<bf16_t, D_, 2>;                \
    case 4: return &layer::launch<bf16_t, D_, 4>;                \
    default: return nullptr;                                    \
    }
    (void)cq1; (void)ck1; (void)cq2; (void)ck2;
    if (d == 32) { MTA_LAYER_CH(32) }
    if (d == 64) { MTA_LAYER_CH(64) }
    if (d == 128) { MTA_LAYER_CH(128) }
#undef MTA_LAYER_CH
    return nullptr;
}

}  // namespace mta
