// mta_bwd_gen_api.h — host interface of the backward pass for every
// placement (kernels in mta_bwd_gen.h, launch sequence in
// mta_inst_bwd_gen.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace mta {
namespace gen {

struct GenArgs {
    const void *q, *k, *v, *dout;
    const float *theta, *w, *gn_w, *gn_b, *gate;
    float *dq, *dk, *dv, *dtheta, *dw, *dgn_w, *dgn_b, *dgate;
    int B, H, T, d, c_q, c_k, c_h, kq_place, head_place, bf16;
    float eps, depth_scale;
};

constexpr int MAX_T = 1 << 15;  // one head's map is then at most 4 GiB
constexpr size_t CHUNK_CAP = (size_t)16 << 30;

// Map slots used by a placement (see the slot plan in the launcher).
int n_slots(int kq_place, int head_place);
// Bytes one unit (head group) needs; a workspace holds whole units.
size_t unit_bytes(int T, int d, int c_h, int kq_place, int head_place);
// The workspace the library asks for: all units at once, or as many as fit
// CHUNK_CAP (at least one).
size_t workspace_bytes(int B, int H, int T, int d, int c_h, int kq_place, int head_place);
hipError_t backward(const GenArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

}  // namespace gen
}  // namespace mta
