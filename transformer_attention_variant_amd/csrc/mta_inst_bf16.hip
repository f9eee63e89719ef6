// bfloat16 kernels: compile-time stencils at d=128 for the kernel sizes of the
// 2K/4K/8K workloads (4x9, 6x11, 8x15) and 1x1; every other size is
// runtime-sized.
#include "mta_launch.h"

namespace mta {
#define ELT bf16_t
#define MTA_FIND_NAME find_launch_bf16
#define FAST_LIST(X) X(128, 1, 1) X(128, 4, 9) X(128, 6, 11) X(128, 8, 15)
#include "mta_inst.inc"
}  // namespace mta
