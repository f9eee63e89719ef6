// Head-split kernels (bf16, d = 128, head mix after the softmax) for
// the kernel sizes of the 2K/4K/8K workloads, 8x13 and 1x1: one pass with the
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
    MTA_V4_SIZE(8, 13)
    MTA_V4_SIZE(8, 15)
    return nullptr;
}

// Head groups of one head (c_h = 1), two per workgroup: one pass with the
// key-query convolution before the softmax (either form), two passes with it
// after the softmax; the caller counts head pairs in p.G.
#define MTA_V4N_SIZE(CQ_, CK_)                                                                         \
    if (cq == CQ_ && ck == CK_)                                                                        \
        return post ? &v4::launch<CQ_, CK_, false, true, false, true>                                 \
                    : (exact ? &v4::launch<CQ_, CK_, true, false, false, true>                        \
                             : &v4::launch<CQ_, CK_, false, false, false, true>);

LaunchFn find_launch_v4_pairs(int d, int cq, int ck, int post, int exact)
{
    if (d != 128 || (post && exact)) return nullptr;
    MTA_V4N_SIZE(1, 1)
    MTA_V4N_SIZE(4, 9)
    MTA_V4N_SIZE(6, 11)
    MTA_V4N_SIZE(8, 13)
    MTA_V4N_SIZE(8, 15)
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

// Groups of 4, 8 or 16 heads, one workgroup per output head pair sweeping the
// group's source pairs; either key-query placement; the caller counts output
// pairs in p.G and source pairs per group in p.npair.  f16pv: P.V with fp16
// operands (groups of 8 and 16).
#define MTA_V4Q_SIZE(CQ_, CK_, PPL_)                                                                   \
    if (cq == CQ_ && ck == CK_)                                                                        \
        return post ? &v4::launch<CQ_, CK_, false, true, false, false, true, PPL_>                    \
                    : (exact ? &v4::launch<CQ_, CK_, true, false, false, false, true, PPL_>           \
                             : &v4::launch<CQ_, CK_, false, false, false, false, true, PPL_>);
#define MTA_V4Q_SIZES(PPL_)        \
    MTA_V4Q_SIZE(1, 1, PPL_)       \
    MTA_V4Q_SIZE(4, 9, PPL_)       \
    MTA_V4Q_SIZE(6, 11, PPL_)      \
    MTA_V4Q_SIZE(8, 13, PPL_)      \
    MTA_V4Q_SIZE(8, 15, PPL_)

LaunchFn find_launch_v4_quad(int d, int cq, int ck, int post, int exact, int f16pv)
{
    if (d != 128 || (post && exact)) return nullptr;
    if (f16pv) {
        MTA_V4Q_SIZES(true)
    } else {
        MTA_V4Q_SIZES(false)
    }
    return nullptr;
}

}  // namespace mta
