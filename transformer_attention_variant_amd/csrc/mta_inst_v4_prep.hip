// Gradient-preparation variants of the one-pass head-split kernels (the
// head-split forward with the epilogue of the backward's first kernel) for the
// kernel sizes of the 2K/4K/8K workloads and 1x1.
#include "mta_fwd_v4.h"
#include "mta_launch.h"

namespace mta {

#define MTA_V4P_SIZE(CQ_, CK_) \
    if (cq == CQ_ && ck == CK_) return exact ? &v4::launch_prep<CQ_, CK_, true> : &v4::launch_prep<CQ_, CK_, false>;

PrepFn find_launch_v4_prep(int d, int ch, int cq, int ck, int exact)
{
    if (d != 128 || ch != 2) return nullptr;
    MTA_V4P_SIZE(1, 1)
    MTA_V4P_SIZE(4, 9)
    MTA_V4P_SIZE(6, 11)
    MTA_V4P_SIZE(8, 13)
    MTA_V4P_SIZE(8, 15)
    return nullptr;
}

}  // namespace mta
