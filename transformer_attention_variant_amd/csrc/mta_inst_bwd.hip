// Backward kernels (mta_bwd.h): float32 and bfloat16, d in {32, 64, 128},
// c_h in {1, 2}; runtime-sized stencils, compile-time 4x9, 6x11 and 8x15 for
// the bf16 workloads (d = 128, c_h = 2).
#include "mta_bwd.h"

namespace mta {
namespace bwd {

// grid_a = 0: the first kernel's outputs come from elsewhere (the head-split
// forward's gradient-preparation variant); only the main kernel runs.
template <typename DT, int D, int CH, int CQ, int CK, int EXM = 0>
hipError_t launch(const BParams &p, int grid_a, size_t lds_a, int grid_b, size_t lds_b, hipStream_t s)
{
    auto fa = mta_bwd_prep<DT, D, CH, CQ, CK>;
    auto fb = mta_bwd_main<DT, D, CH, CQ, CK, EXM>;
    hipError_t e;
    if (grid_a > 0) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(fa), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds_a);
        if (e != hipSuccess) return e;
    }
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fb), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_b);
    if (e != hipSuccess) return e;
    if (grid_a > 0) {
        hipLaunchKernelGGL(fa, dim3(grid_a), dim3(NT), lds_a, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fb, dim3(grid_b), dim3(NTB), lds_b, s, p);
    return hipGetLastError();
}

}  // namespace bwd

bool bwd_fixed_sizes(int dtype_bf16, int d, int ch, int cq, int ck)
{
    return dtype_bf16 && d == 128 && ch == 2 && ((cq == 6 && ck == 11) || (cq == 4 && ck == 9) || (cq == 8 && ck == 15));
}

bwd::BwdFn find_launch_bwd(int dtype_bf16, int d, int ch, int cq, int ck, int exact)
{
    using namespace bwd;
    if (bwd_fixed_sizes(dtype_bf16, d, ch, cq, ck)) {
        // the masking form fixed at compile time (two-pass masks: the kernel
        // gradient and the transposed stencil on the matrix cores)
        if (cq == 6) return exact ? &launch<bf16_t, 128, 2, 6, 11, 2> : &launch<bf16_t, 128, 2, 6, 11, 1>;
        if (cq == 4) return exact ? &launch<bf16_t, 128, 2, 4, 9, 2> : &launch<bf16_t, 128, 2, 4, 9, 1>;
        return exact ? &launch<bf16_t, 128, 2, 8, 15, 2> : &launch<bf16_t, 128, 2, 8, 15, 1>;
    }
#define MTA_BWD_D(T_, D_)                                          \
    if (d == D_) {                                                 \
        if (ch == 1) return &launch<T_, D_, 1, 0, 0>;              \
        if (ch == 2) return &launch<T_, D_, 2, 0, 0>;              \
        return nullptr;                                            \
    }
    if (dtype_bf16) {
        MTA_BWD_D(bf16_t, 32)
        MTA_BWD_D(bf16_t, 64)
        MTA_BWD_D(bf16_t, 128)
    } else {
        MTA_BWD_D(float, 32)
        MTA_BWD_D(float, 64)
        MTA_BWD_D(float, 128)
    }
#undef MTA_BWD_D
    return nullptr;
}

// Clears the float buffers the kernels accumulate into (a kernel, so that the
// call can be captured in a graph).
__global__ void mta_fill_zero(bwd::ZeroList z)
{
    for (int k = 0; k < z.k; ++k) {
        float *p = z.p[k];
        const size_t c = z.n[k];
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < c; i += (size_t)gridDim.x * blockDim.x)
            p[i] = 0.f;
    }
}

hipError_t launch_fill_zero(const bwd::ZeroList &z, hipStream_t s)
{
    hipLaunchKernelGGL(mta_fill_zero, dim3(1024), dim3(256), 0, s, z);
    return hipGetLastError();
}

}  // namespace mta
