// The repeated convolution's head-split kernel (mta_fwd_rep.h) for the kernel
// sizes of the 4K workload's repeated form (6x11 before and after the
// softmax), the 8K sweep's 4x9, and 1x1 (the contraction alone, against which
// the convolution stages are measured).
#include "mta_fwd_rep.h"

namespace mta {
namespace rep {

size_t lds_bytes(int cq1, int ck1, int cq2, int ck2)
{
    if (cq1 == 6 && ck1 == 11 && cq2 == 6 && ck2 == 11) return (size_t)rlayout<6, 11, 6, 11>().total;
    if (cq1 == 4 && ck1 == 9 && cq2 == 4 && ck2 == 9) return (size_t)rlayout<4, 9, 4, 9>().total;
    if (cq1 == 1 && ck1 == 1 && cq2 == 1 && ck2 == 1) return (size_t)rlayout<1, 1, 1, 1>().total;
    return 0;
}

RepFn find_launch(int d, int ch, int cq1, int ck1, int cq2, int ck2)
{
    if (d != 128 || ch != 2) return nullptr;
    if (cq1 == 6 && ck1 == 11 && cq2 == 6 && ck2 == 11) return &launch<6, 11, 6, 11>;
    if (cq1 == 4 && ck1 == 9 && cq2 == 4 && ck2 == 9) return &launch<4, 9, 4, 9>;
    if (cq1 == 1 && ck1 == 1 && cq2 == 1 && ck2 == 1) return &launch<1, 1, 1, 1>;
    return nullptr;
}

}  // namespace rep
}  // namespace mta
