// float32 kernels: compile-time stencils for the kernel sizes of the fp32
// workloads (3x5 at d=32, 2x9 at d=64); every other size is runtime-sized.
#include "mta_launch.h"

namespace mta {
#define ELT float
#define MTA_FIND_NAME find_launch_f32
#define FAST_LIST(X) X(32, 3, 5) X(64, 2, 9)
#include "mta_inst.inc"
}  // namespace mta
