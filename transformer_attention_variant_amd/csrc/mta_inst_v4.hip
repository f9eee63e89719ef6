// Head-split kernels (bf16, d = 128, c_h = 2, head mix after the softmax) for
// the kernel sizes of the 2K/4K/8K workloads and 1x1: one pass with the
// key-query convolution before the softmax (either form), two passes with it
// after the softmax.
#include "mta_fwd_v4.h"
#include "mta_launch.h"

namespace mta {

#define MTA_V4_SIZE(CQ_, CK_)                                                                          \
    if (cq == CQ_ && ck == CK_)                                                                        \
        return post ? &v4::launch<CQ_, CK_, false, true>                                              \
                    : (exact ? &v4::launch<CQ_, CK_, true> : &v4::launch<CQ_, CK_, false>);

LaunchFn find_launch_v4(int d, int ch, int cq, int ck, int post, int exact, int hpre)
{
    if (d != 128 || ch != 2 || hpre || (post && exact)) return nullptr;
    MTA_V4_SIZE(1, 1)
    MTA_V4_SIZE(4, 9)
    MTA_V4_SIZE(6, 11)
    MTA_V4_SIZE(8, 15)
    return nullptr;
}

// The 3D form (both-pre-softmax 3D convolution, no head mix) at the 4K
// workload's kernel size and 1x1.
LaunchFn find_launch_v4_3d(int d, int ch, int cq, int ck)
{
    if (d != 128 || ch != 2) return nullptr;
    if (cq == 6 && ck == 11) return &v4::launch<6, 11, false, false, true>;
    if (cq == 1 && ck == 1) return &v4::launch<1, 1, false, false, true>;
    return nullptr;
}

}  // namespace mta
