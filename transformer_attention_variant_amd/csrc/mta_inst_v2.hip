// Pipelined 8-wave kernels (bf16, d = 128, head mix after the softmax) for the
// kernel sizes of the 2K/4K/8K workloads and 1x1.
#include "mta_fwd_v2.h"
#include "mta_launch.h"

namespace mta {

#define MTA_V2_L(CH_, CQ_, CK_, MS_) \
    (post ? &v2::launch<128, CH_, CQ_, CK_, true, MS_> : &v2::launch<128, CH_, CQ_, CK_, false, MS_>)
#define MTA_V2_SIZE(CQ_, CK_, MS_)                           \
    if (cq == CQ_ && ck == CK_) {                            \
        switch (ch) {                                        \
        case 1: return MTA_V2_L(1, CQ_, CK_, MS_);           \
        case 2: return MTA_V2_L(2, CQ_, CK_, MS_);           \
        case 4: return MTA_V2_L(4, CQ_, CK_, MS_);           \
        default: return nullptr;                             \
        }                                                    \
    }

// ms = 1: stencil on the matrix cores (needs c_k <= 17); ms = 0: fp32 VALU stencil.
LaunchFn find_launch_v2(int d, int ch, int cq, int ck, int post, int hpre, int ms)
{
    if (d != 128 || hpre) return nullptr;
    if (ms) {
        MTA_V2_SIZE(1, 1, true)
        MTA_V2_SIZE(4, 9, true)
        MTA_V2_SIZE(6, 11, true)
        MTA_V2_SIZE(8, 15, true)
    } else {
        MTA_V2_SIZE(1, 1, false)
        MTA_V2_SIZE(4, 9, false)
        MTA_V2_SIZE(6, 11, false)
        MTA_V2_SIZE(8, 15, false)
    }
    return nullptr;
}

}  // namespace mta
