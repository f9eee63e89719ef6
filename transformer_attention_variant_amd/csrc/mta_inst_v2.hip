// Pipelined 8-wave kernels (bf16, d = 128, head mix after the softmax) for the
// kernel sizes of the 2K/4K/8K workloads and 1x1: two-pass masking and the
// post-softmax convolution.  The exact-indicator variants are in
// mta_inst_v2_exact.hip; find_launch_v2 picks between the two tables.
#include "mta_fwd_v2.h"
#include "mta_launch.h"

namespace mta {

LaunchFn find_launch_v2_exact(int ch, int cq, int ck, int ms);

namespace {
#define MTA_V2_POST(CH_, CQ_, CK_, MS_) \
    (post ? &v2::launch<128, CH_, CQ_, CK_, true, MS_, false> : nullptr)
#define MTA_V2_ANY(CH_, CQ_, CK_, MS_)                                  \
    (post ? &v2::launch<128, CH_, CQ_, CK_, true, MS_, false>          \
          : &v2::launch<128, CH_, CQ_, CK_, false, MS_, false>)
#define MTA_V2_PICK pick_two_pass
#define MTA_V2_FIND find_two_pass
#include "mta_inst_v2.inc"
}  // namespace

LaunchFn find_launch_v2(int d, int ch, int cq, int ck, int post, int exact, int hpre, int ms)
{
    if (d != 128 || hpre) return nullptr;
    return exact ? find_launch_v2_exact(ch, cq, ck, ms) : find_two_pass(ch, cq, ck, post, ms);
}

}  // namespace mta
