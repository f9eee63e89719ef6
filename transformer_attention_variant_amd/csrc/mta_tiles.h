// mta_tiles.h — LDS layout helpers of the head-split kernels: swizzles of the
// DMA-written Q, K and V tiles, the transposing V read, and the barrier that
// publishes LDS writes only.
#pragma once

#include "mta_fwd_kernel.h"

namespace mta {
namespace tile {

// ---------------------------------------------------------------------------
// Q, K and V tiles (d = 128: rows of 256 bytes, 16 chunks of 16 bytes) are
// written by the DMA form of the global load (global_load_lds_dwordx4: lane i
// of a wave puts its 16 bytes at base + 16 i), so rows carry no padding;
// instead the chunks of row r are stored in the order c ^ swz(r).  gfx950's
// LDS has 64 banks of 4 bytes; ds_read_b128 serves a wave in four passes of 16
// lanes (the pass of lane 0 holds lanes 0-3, 12-15 and 20-27), and the
// transposing read of a 16-row V block keeps rows r and r + 8 apart.  With the
// swizzles below every pass of the fragment reads and of the V reads touches
// each bank once (checked with the bank-conflict counter).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_void_p;
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_p;

__device__ inline int swz_k(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ inline int swz_v(int r) { return 2 * (r & 7); }

// Workgroup barrier that publishes LDS writes but lets this wave's DMA tile
// loads stay in flight (a __syncthreads() fence would wait for them too).
// Only valid where no wave reads the DMA targets before the next full barrier,
// which waits for them.
__device__ inline void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposing read of the swizzled V tile (ds_read_b64_tr_b16): within each
// 16-lane group, element e = 0..3 of lane i is the (i mod 4)-th element of the
// 4-element row that lane 4e + i/4 addresses.  Lane j addresses
// V[kb + j/4][d0 + 4(j mod 4)], so lane i receives V[kb + e][d0 + i]: four
// consecutive keys of its own d column, the B operand of the P.V product.
__device__ inline s16x4 vread_tr4(const bf16_t *vbuf, int kb, int d0, int j)
{
    const int row = kb + (j >> 2), col = d0 + 4 * (j & 3);
    const bf16_t *a = vbuf + row * 128 + 8 * ((col >> 3) ^ swz_v(row)) + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(a));
}

}  // namespace tile
}  // namespace mta
