// General-layer kernels, float32 (d in {32, 64, 128}, c_h in {1, 2, 4}).
#include "mta_fwd_layer.h"

namespace mta {

// cq1/ck1: pre-softmax kernel size (0 without one); cq2/ck2: post-softmax one.
layer::LayerFn find_launch_layer_f32(int d, int ch, int cq1, int ck1, int cq2, int ck2)
{
#define MTA_LAYER_CH(D_)                                        \
    switch (ch) {                                               \
    case 1: return &layer::launch<float, D_, 1>;                \
    case 2: return &layer::launch<float, D_, 2>;                \
    case 4: return &layer::launch<float, D_, 4>;                \
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
