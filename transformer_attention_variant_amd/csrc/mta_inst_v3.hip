// One-pass key-split kernels (bf16, d = 128, key-query convolution before the
// softmax in either form, head mix after it) for groups of one head (groups of
// two run the head-split kernel of mta_fwd_v4.h), for the kernel sizes of the
// 2K/4K/8K workloads and 1x1.
#include "mta_fwd_v3.h"
#include "mta_launch.h"

namespace mta {

#define MTA_V3_L(CH_, CQ_, CK_) \
    (exact ? &v3::launch<128, CH_, CQ_, CK_, true> : &v3::launch<128, CH_, CQ_, CK_, false>)
#define MTA_V3_SIZE(CQ_, CK_)                            \
    if (cq == CQ_ && ck == CK_) {                        \
        if (ch == 1) return MTA_V3_L(1, CQ_, CK_);       \
        return nullptr;                                  \
    }

LaunchFn find_launch_v3(int d, int ch, int cq, int ck, int post, int exact, int hpre)
{
    if (d != 128 || post || hpre) return nullptr;
    MTA_V3_SIZE(1, 1)
    MTA_V3_SIZE(4, 9)
    MTA_V3_SIZE(6, 11)
    MTA_V3_SIZE(8, 15)
    return nullptr;
}

}  // namespace mta
