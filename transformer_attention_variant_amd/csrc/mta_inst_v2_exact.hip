// Pipelined 8-wave kernels with the key-query convolution before the softmax
// in the exact form of Eq. 4 (its causal indicator instead of the two-pass
// masks), for the same kernel sizes as mta_inst_v2.hip.
#include "mta_fwd_v2.h"
#include "mta_launch.h"

namespace mta {

namespace {
#define MTA_V2_POST(CH_, CQ_, CK_, MS_) (LaunchFn) nullptr
#define MTA_V2_ANY(CH_, CQ_, CK_, MS_) (&v2::launch<128, CH_, CQ_, CK_, false, MS_, true>)
#define MTA_V2_PICK pick_exact
#define MTA_V2_FIND find_exact
#include "mta_inst_v2.inc"
}  // namespace

LaunchFn find_launch_v2_exact(int ch, int cq, int ck, int ms) { return find_exact(ch, cq, ck, 0, ms); }

}  // namespace mta
