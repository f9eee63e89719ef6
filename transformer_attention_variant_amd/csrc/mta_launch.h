// mta_launch.h — launch helpers shared by the instantiation units and the ABI.
#pragma once

#include "mta_fwd_kernel.h"

namespace mta {

typedef hipError_t (*LaunchFn)(const Params &p, int grid, size_t lds, hipStream_t s);

template <typename DT, int D, int CH, int CQ, int CK, bool POST, bool HPRE>
hipError_t launch(const Params &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_kernel<DT, D, CH, CQ, CK, POST, HPRE>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p);
    return hipGetLastError();
}

// Kernel lookup per element type; null when (d, c_h) is not instantiated.
// Kernel sizes (c_q, c_k) with a compile-time stencil get it when the head mix
// follows the softmax; every other case runs the runtime-sized stencil of the
// same kernel template.
LaunchFn find_launch_f32(int d, int ch, int cq, int ck, int post, int hpre);
LaunchFn find_launch_bf16(int d, int ch, int cq, int ck, int post, int hpre);
// General-layer kernels (mta_fwd_layer.h) per element type; null when (d, c_h)
// is not instantiated.
namespace layer {
struct LParams;
typedef hipError_t (*LayerFn)(const LParams &p, int grid, size_t lds, hipStream_t s);
}  // namespace layer
layer::LayerFn find_launch_layer_f32(int d, int ch, int cq1, int ck1, int cq2, int ck2);
layer::LayerFn find_launch_layer_bf16(int d, int ch, int cq1, int ck1, int cq2, int ck2);
// Head-split bf16 kernels for c_h = 2 (mta_fwd_v4.h); null when not instantiated.
LaunchFn find_launch_v4(int d, int ch, int cq, int ck, int post, int exact, int hpre);
// Its form for head groups of one head, two groups per workgroup (p.G counts
// head pairs); null when not instantiated.
LaunchFn find_launch_v4_pairs(int d, int cq, int ck, int post, int exact);
// Its 3D-convolution form (two-pass masks, no head mix); null when not instantiated.
LaunchFn find_launch_v4_3d(int d, int ch, int cq, int ck);
// Groups of 4, 8 or 16 heads: the head-split kernel per output head pair, one
// sweep per source pair (p.G counts output pairs, p.npair source pairs per
// group); f16pv: P.V with fp16 operands.  Null when not instantiated.
LaunchFn find_launch_v4_quad(int d, int cq, int ck, int post, int exact, int f16pv);
// Their gradient-preparation variants (key-query convolution before the
// softmax, head mix after it); null when not instantiated.
namespace v4 {
struct PrepArgs;
}
typedef hipError_t (*PrepFn)(const Params &p, const v4::PrepArgs &pa, int grid, size_t lds, hipStream_t s);
PrepFn find_launch_v4_prep(int d, int ch, int cq, int ck, int exact);

}  // namespace mta
