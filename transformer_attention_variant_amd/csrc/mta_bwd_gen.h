// mta_bwd_gen.h — the backward pass for every placement of the two
// convolutions, with each head's T x T maps held in a device workspace.
//
// Forward (page "Multi-Token Attention — Paper Graph", section 3.4), per head:
//   S  = Q K^T / sqrt(d)                                    ("Standard Multi-Head Attention")
//   C  = Eq. 4 on Mask_0(S) (two-pass) or on S with Eq. 4's indicator, if the
//        key-query convolution precedes the softmax; else C = S ("Key-Query Convolution")
//   L  = the head mix of C (Eq. 7 on logits) if it precedes the softmax; else C
//   P  = softmax(Mask_-inf(L))
//   P2 = Mask_0(Eq. 4 on P) if the key-query convolution follows the softmax; else P
//   P3 = the head mix of P2 (Eq. 7) if it follows the softmax; else P2
//   O  = P3 V,  y = scale_h (gamma (O - mu) / sigma + beta),
//        scale_h = depth_scale [x sigmoid(g_h)]     ("Group Normalization with Sigmoid Gating")
// Backward, the chain rule taken stage by stage in reverse:
//   GroupNorm -> dO, dgamma, dbeta, dgate;  dP3 = dO V^T, dV = P3^T dO;
//   head mix after the softmax: dP2^b = sum_a w_ab dP3^a, dw_ab = sum dP3^a P2^b;
//   convolution after it: dP = (transposed Eq. 4)(Mask_0 dP2), dtheta = sum Mask_0(dP2) x shifted P;
//   softmax: dL = P (dP - sum_j P dP);
//   head mix before it: dC^b = sum_a w_ab dL^a, dw_ab = sum dL^a C^b;
//   convolution before it: dS = (transposed Eq. 4 with the same masks or indicator)(dC),
//   dtheta = sum dC x shifted input;  dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
//
// Layout: maps are float32 [unit][c_h][Tp][Tp] (Tp = T rounded up to 64) in
// "slots" of the workspace; only band tiles are touched — the 64 x 64 tiles
// of the causal triangle plus the tile right of the diagonal one, which Eq. 4's
// indicator reaches (keys up to c_q - 1 past a row).  Every kernel writes
// every element of the band tiles it produces (zero where the map is zero),
// and reads only elements that some kernel wrote.  Head groups are processed
// in chunks that fit the workspace.  All arithmetic keeps float32 precision:
// products on the matrix cores with fp32 operands (v_mfma_f32_16x16x4_f32) or,
// for bf16 inputs, with bf16 operands whose float32 side is split into three
// bf16 parts (v_mfma_f32_16x16x32_bf16); the stencils, softmax and GroupNorm
// on the VALU in float32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mta_fwd_kernel.h"
#include "mta_bwd_gen_api.h"

namespace mta {
namespace gen {

constexpr int TB = 64;        // map tile edge
constexpr int NTH = 256;      // threads per workgroup
constexpr int XP = 100;       // LDS pitch of a stencil input region: 64 + 31 columns, padded so
                              // that the window reads (rows of 4 lanes x 16 B) hit distinct banks
constexpr int WIN = 48;       // register window of a stencil row: 16 outputs + up to 31 taps

enum Place { KQ_PRE = 0, KQ_POST = 1, KQ_EXACT = 2 };
enum Mode { M_PRE = 0, M_EXACT = 1, M_POST = 2 };    // how a stencil reads its input map

struct GParams {
    const void *q, *k, *v, *dout;     // [B][H][T][d], the call's dtype
    const float *theta, *w, *gn_w, *gn_b, *gate;
    float *dq, *dk, *dv, *dtheta, *dw, *dgn_w, *dgn_b, *dgate;
    int B, H, T, d, c_q, c_k, c_h, G;
    int kq_place, head_place;
    float eps, depth_scale, inv_sqrt_d;
    int Tp, nt, n_band;               // padded T, tiles per side, band tiles per head
    int u0, nu;                       // this chunk: units [u0, u0 + nu)
    float *obuf;                      // [nu][c_h][T][d]: O, then dO
};

// Band tile t of one head -> (row tile, column tile): the triangle jt <= it
// first (row by row), then the tiles (it, it + 1).
__device__ inline void band_tile(int t, int nt, int &it, int &jt)
{
    const int ntri = nt * (nt + 1) / 2;
    if (t < ntri) {
        int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
        if ((i + 1) * (i + 2) / 2 <= t) ++i;
        if (i * (i + 1) / 2 > t) --i;
        it = i;
        jt = t - i * (i + 1) / 2;
    } else {
        it = t - ntri;
        jt = it + 1;
    }
}

// Head bookkeeping for a grid row y = uu * c_h + a of this chunk.
struct HeadIx {
    int uu, a, b, g, h;
};
__device__ inline HeadIx head_ix(const GParams &p, int y)
{
    HeadIx x;
    x.uu = y / p.c_h;
    x.a = y - x.uu * p.c_h;
    const int u = p.u0 + x.uu;
    x.b = u / p.G;
    x.g = u - x.b * p.G;
    x.h = x.g * p.c_h + x.a;
    return x;
}

__device__ inline float *map_of(float *slot, const GParams &p, int y)
{
    return slot + (size_t)y * p.Tp * p.Tp;
}

__device__ inline size_t tensor_off(const GParams &p, const HeadIx &x)
{
    return ((size_t)x.b * p.H + x.h) * (size_t)p.T * p.d;
}

template <typename T>
__device__ inline float to_f(T x)
{
    return (float)x;
}

// Loads 4 consecutive elements as float32.
__device__ inline float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ inline float4 load4(const bf16_t *p)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

__device__ inline f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Sums 16 per-lane partials over the wave: afterwards lane l holds the total
// of partial number ((l >> 2) & 15) (lanes with equal (l >> 2) agree).
// 8 + 4 + 2 + 1 exchanges halve the partials a lane carries while doubling
// the lanes each one is summed over, then two more fold the last 4 lanes.
__device__ inline float reduce16(float (&v)[16], int lane)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const bool up = lane & 32;
        const float send = up ? v[t] : v[t + 8];
        const float keep = up ? v[t + 8] : v[t];
        v[t] = keep + __shfl_xor(send, 32);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool up = lane & 16;
        const float send = up ? v[t] : v[t + 4];
        const float keep = up ? v[t + 4] : v[t];
        v[t] = keep + __shfl_xor(send, 16);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const bool up = lane & 8;
        const float send = up ? v[t] : v[t + 2];
        const float keep = up ? v[t + 2] : v[t];
        v[t] = keep + __shfl_xor(send, 8);
    }
    {
        const bool up = lane & 4;
        const float send = up ? v[0] : v[1];
        const float keep = up ? v[1] : v[0];
        v[0] = keep + __shfl_xor(send, 4);
    }
    float s = v[0];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    return s;
}
// The partial index reduce16 leaves in lane l.
__device__ inline int reduce16_slot(int lane)
{
    return ((lane & 32) ? 8 : 0) + ((lane & 16) ? 4 : 0) + ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
}

// ---------------------------------------------------------------------------
// Products on the matrix cores (fp32 operands, fp32 accumulation).
//
// Operand sources: a [B][H][T][d] tensor of the call's dtype, or the chunk's
// fp32 [nu][c_h][T][d] buffer (O / dO).
enum Src { SRC_TENSOR = 0, SRC_OBUF = 1 };

template <typename DT, int SRC>
__device__ inline const void *rows_base(const GParams &p, const void *tensor, const HeadIx &x, int y)
{
    if (SRC == SRC_OBUF) return p.obuf + (size_t)y * p.T * p.d;
    return static_cast<const DT *>(tensor) + tensor_off(p, x);
}

// Stages rows [r0, r0 + 64) x columns [c0, c0 + W) of a row-major [T][D]
// operand as fp32 into LDS with the given pitch (rows >= T are zero).
template <typename ET, int D, int W = D>
__device__ inline void stage_rows(float *dst, int pitch, const ET *src, int r0, int T, int tid, int c0 = 0)
{
    for (int idx = tid; idx < TB * W / 4; idx += NTH) {
        const int r = idx / (W / 4), c4 = idx - r * (W / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + r < T) x = load4(src + (size_t)(r0 + r) * D + c0 + 4 * c4);
        *reinterpret_cast<float4 *>(dst + r * pitch + 4 * c4) = x;
    }
}

// Stages a 64 x 64 tile of a map (rows i0.., columns j0..) into LDS.
__device__ inline void stage_tile(float *dst, int pitch, const float *map, int Tp, int i0, int j0, int tid)
{
    for (int idx = tid; idx < TB * TB / 4; idx += NTH) {
        const int r = idx >> 4, c4 = idx & 15;
        *reinterpret_cast<float4 *>(dst + r * pitch + 4 * c4) =
            load4(map + (size_t)(i0 + r) * Tp + j0 + 4 * c4);
    }
}

// Register-staged copies of the same two loads, so that the next tile's
// global reads are in flight while the current tile is multiplied.
template <typename ET, int D>
struct RowRegs {
    float4 v[TB * D / 4 / NTH];
    __device__ void load(const ET *src, int r0, int T, int tid)
    {
#pragma unroll
        for (int k = 0; k < TB * D / 4 / NTH; ++k) {
            const int idx = tid + k * NTH, r = idx / (D / 4), c4 = idx - r * (D / 4);
            v[k] = r0 + r < T ? load4(src + (size_t)(r0 + r) * D + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    __device__ void store(float *dst, int pitch, int tid) const
    {
#pragma unroll
        for (int k = 0; k < TB * D / 4 / NTH; ++k) {
            const int idx = tid + k * NTH, r = idx / (D / 4), c4 = idx - r * (D / 4);
            *reinterpret_cast<float4 *>(dst + r * pitch + 4 * c4) = v[k];
        }
    }
};

struct TileRegs {
    float4 v[TB * TB / 4 / NTH];
    __device__ void load(const float *map, int Tp, int i0, int j0, int tid)
    {
#pragma unroll
        for (int k = 0; k < TB * TB / 4 / NTH; ++k) {
            const int idx = tid + k * NTH, r = idx >> 4, c4 = idx & 15;
            v[k] = load4(map + (size_t)(i0 + r) * Tp + j0 + 4 * c4);
        }
    }
    __device__ void store(float *dst, int pitch, int tid) const
    {
#pragma unroll
        for (int k = 0; k < TB * TB / 4 / NTH; ++k) {
            const int idx = tid + k * NTH, r = idx >> 4, c4 = idx & 15;
            *reinterpret_cast<float4 *>(dst + r * pitch + 4 * c4) = v[k];
        }
    }
};

// M[i][j] = alpha sum_c A[i][c] B[j][c] on every band tile (grid: n_band x
// heads of the chunk).  A: Q (SRC_TENSOR) or dO (SRC_OBUF); B: K or V.
template <typename DT, int D, int SRCA>
__global__ void __launch_bounds__(NTH) gen_gemm_nt(GParams p, const void *a_tensor, const void *b_tensor,
                                                   float *slot, float alpha)
{
    typedef typename std::conditional<SRCA == SRC_OBUF, float, DT>::type AT;
    constexpr int KC = D < 64 ? D : 64;  // d columns staged at a time
    constexpr int AP = KC + 4;
    __shared__ __align__(16) float As[TB * AP];
    __shared__ __align__(16) float Bs[TB * AP];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB, j0 = jt * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const AT *asrc = static_cast<const AT *>(rows_base<DT, SRCA>(p, a_tensor, x, y));
    const DT *bsrc = static_cast<const DT *>(rows_base<DT, SRC_TENSOR>(p, b_tensor, x, y));
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
    const int lr = lane & 15, lk = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < D; c0 += KC) {
        if (c0) __syncthreads();
        stage_rows<AT, D, KC>(As, AP, asrc, i0, p.T, tid, c0);
        stage_rows<DT, D, KC>(Bs, AP, bsrc, j0, p.T, tid, c0);
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < KC; kk += 4) {
            const float a0 = As[(wr + lr) * AP + kk + lk], a1 = As[(wr + 16 + lr) * AP + kk + lk];
            const float b0 = Bs[(wc + lr) * AP + kk + lk], b1 = Bs[(wc + 16 + lr) * AP + kk + lk];
            acc[0][0] = mfma4(a0, b0, acc[0][0]);
            acc[0][1] = mfma4(a0, b1, acc[0][1]);
            acc[1][0] = mfma4(a1, b0, acc[1][0]);
            acc[1][1] = mfma4(a1, b1, acc[1][1]);
        }
    }
    float *m = map_of(slot, p, y);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + wr + 16 * mb + 4 * lk + r, j = j0 + wc + 16 * nb + lr;
                m[(size_t)i * p.Tp + j] = alpha * acc[mb][nb][r];
            }
}

// Out[i][:] = alpha sum_j M[i][j] B[j][:] for the rows of row tile
// nt - 1 - blockIdx.x, j over the band (grid: nt x heads).  Out: the chunk's O buffer or a
// [B][H][T][d] fp32 gradient tensor.
template <typename DT, int D, bool TO_OBUF>
__global__ void __launch_bounds__(NTH) gen_gemm_mn(GParams p, const float *slot, const void *b_tensor, float *out,
                                                   float alpha)
{
    constexpr int MP = TB + 4, BP = D + 16;
    __shared__ __align__(16) float Ms[TB * MP];
    __shared__ __align__(16) float Bs[TB * BP];
    const int it = p.nt - 1 - (int)blockIdx.x, y = blockIdx.y;  // the longest rows first
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const float *m = map_of(const_cast<float *>(slot), p, y);
    const DT *bsrc = static_cast<const DT *>(b_tensor) + tensor_off(p, x);
    f32x4 acc[D / 16];
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int jt_end = it + 1 < p.nt ? it + 1 : p.nt - 1;
    TileRegs mr;
    RowRegs<DT, D> br;
    mr.load(m, p.Tp, i0, 0, tid);
    br.load(bsrc, 0, p.T, tid);
    for (int jt = 0; jt <= jt_end; ++jt) {
        mr.store(Ms, MP, tid);
        br.store(Bs, BP, tid);
        __syncthreads();
        if (jt < jt_end) {  // the next tile's reads overlap this tile's products
            mr.load(m, p.Tp, i0, (jt + 1) * TB, tid);
            br.load(bsrc, (jt + 1) * TB, p.T, tid);
        }
#pragma unroll 4
        for (int kk = 0; kk < TB; kk += 4) {
            const float a = Ms[(16 * w + lr) * MP + kk + lk];
#pragma unroll
            for (int n = 0; n < D / 16; ++n) acc[n] = mfma4(a, Bs[(kk + lk) * BP + 16 * n + lr], acc[n]);
        }
        __syncthreads();
    }
    float *o = TO_OBUF ? p.obuf + (size_t)y * p.T * D : out + tensor_off(p, x);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * w + 4 * lk + r;
            if (i < p.T) o[(size_t)i * D + 16 * n + lr] = alpha * acc[n][r];
        }
}

// Out[j][:] = alpha sum_i M[i][j] B[i][:] for the keys of column tile
// blockIdx.x (the longest columns first), i over the band (grid: nt x heads); Out a [B][H][T][d] fp32
// gradient tensor.  B: dO (SRC_OBUF) or Q (SRC_TENSOR).
template <typename DT, int D, int SRCB>
__global__ void __launch_bounds__(NTH) gen_gemm_tn(GParams p, const float *slot, const void *b_tensor, float *out,
                                                   float alpha)
{
    typedef typename std::conditional<SRCB == SRC_OBUF, float, DT>::type BT;
    constexpr int MP = TB + 16, BP = D + 16;
    __shared__ __align__(16) float Ms[TB * MP];
    __shared__ __align__(16) float Bs[TB * BP];
    const int jt = blockIdx.x, y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int j0 = jt * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const float *m = map_of(const_cast<float *>(slot), p, y);
    const BT *bsrc = static_cast<const BT *>(rows_base<DT, SRCB>(p, b_tensor, x, y));
    f32x4 acc[D / 16];
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int it0 = jt > 0 ? jt - 1 : 0;
    TileRegs mr;
    RowRegs<BT, D> br;
    mr.load(m, p.Tp, it0 * TB, j0, tid);
    br.load(bsrc, it0 * TB, p.T, tid);
    for (int it = it0; it < p.nt; ++it) {
        mr.store(Ms, MP, tid);
        br.store(Bs, BP, tid);
        __syncthreads();
        if (it + 1 < p.nt) {  // the next tile's reads overlap this tile's products
            mr.load(m, p.Tp, (it + 1) * TB, j0, tid);
            br.load(bsrc, (it + 1) * TB, p.T, tid);
        }
#pragma unroll 4
        for (int kk = 0; kk < TB; kk += 4) {
            const float a = Ms[(kk + lk) * MP + 16 * w + lr];
#pragma unroll
            for (int n = 0; n < D / 16; ++n) acc[n] = mfma4(a, Bs[(kk + lk) * BP + 16 * n + lr], acc[n]);
        }
        __syncthreads();
    }
    float *o = out + tensor_off(p, x);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + 16 * w + 4 * lk + r;
            if (j < p.T) o[(size_t)j * D + 16 * n + lr] = alpha * acc[n][r];
        }
}

// ---------------------------------------------------------------------------
// The same products for bf16 inputs on the 16-bit matrix cores
// (v_mfma_f32_16x16x32_bf16, float32 accumulation).  A bf16 input tensor (Q,
// K, V) is an exact operand; a float32 operand (a map, dO) is split into three
// bf16 parts x = h + m + l (h = bf16(x), m = bf16(x - h), l = bf16(x - h - m):
// 24 significant bits, each remainder below 2^-8 of the previous part), and
// the three parts' products with the exact operand accumulate in float32, so
// the sums keep float32 precision at a third of the 16-bit rate (against an
// eighth for float32 operands).  dV = P3^T dO, whose operands are both
// float32, keeps the float32 products (six split products, staged half of d
// at a time, measured 5% faster for that kernel: not worth the code).

typedef short s16x4g __attribute__((ext_vector_type(4)));
typedef short s16x8g __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4g *lds_s16x4g_p;

// 4 consecutive values into NP bf16 planes (plane k at dst + k * pstride):
// NP = 1 rounds (exact for values that came from bf16), NP = 3 splits.
template <int NP>
__device__ inline void put4_planes(bf16_t *dst, int pstride, float4 v)
{
    const float x[4] = {v.x, v.y, v.z, v.w};
    bf16x4g o[NP];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16_t h = (bf16_t)x[e];
        o[0][e] = h;
        if constexpr (NP == 3) {
            const float r1 = x[e] - (float)h;
            const bf16_t m = (bf16_t)r1;
            o[1][e] = m;
            o[2][e] = (bf16_t)(r1 - (float)m);
        }
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) *reinterpret_cast<bf16x4g *>(dst + k * pstride) = o[k];
}

// Rows [r0, r0 + 64) x columns [c0, c0 + W) of a row-major [T][D] operand into
// NP bf16 planes (pitch in halves; rows >= T are zero).
template <int NP, typename ET, int D, int W>
__device__ inline void stage_rows16(bf16_t *dst, int pitch, const ET *src, int r0, int T, int tid, int c0)
{
    for (int idx = tid; idx < TB * W / 4; idx += NTH) {
        const int r = idx / (W / 4), c4 = idx - r * (W / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + r < T) x = load4(src + (size_t)(r0 + r) * D + c0 + 4 * c4);
        put4_planes<NP>(dst + r * pitch + 4 * c4, TB * pitch, x);
    }
}

// The register-staged loads of gen_gemm_mn / tn, stored as bf16 planes.
template <int NP, typename ET, int D>
__device__ inline void store_rows16(const RowRegs<ET, D> &rr, bf16_t *dst, int pitch, int tid)
{
#pragma unroll
    for (int k = 0; k < TB * D / 4 / NTH; ++k) {
        const int idx = tid + k * NTH, r = idx / (D / 4), c4 = idx - r * (D / 4);
        put4_planes<NP>(dst + r * pitch + 4 * c4, TB * pitch, rr.v[k]);
    }
}
template <int NP>
__device__ inline void store_tile16(const TileRegs &tr, bf16_t *dst, int pitch, int tid)
{
#pragma unroll
    for (int k = 0; k < TB * TB / 4 / NTH; ++k) {
        const int idx = tid + k * NTH, r = idx >> 4, c4 = idx & 15;
        put4_planes<NP>(dst + r * pitch + 4 * c4, TB * pitch, tr.v[k]);
    }
}

// Operand of a 16x16x32 product along rows of a row-major bf16 tile: lane
// (n = lane%16, g = lane/16) gets rows k0 + 8g .. k0 + 8g + 7 of column
// c0 + n, with two transposing reads (ds_read_b64_tr_b16: within each
// 16-lane group, element e of lane i is the (i mod 4)-th element of the
// 4-element row that lane 4e + i/4 addresses; lane j addresses row
// k0 + 8g + j/4, columns c0 + 4(j mod 4)).
__device__ inline bf16x8 tr_frag(const bf16_t *tile, int pitch, int k0, int c0, int lane)
{
    const int j = lane & 15, g = lane >> 4;
    const bf16_t *a = tile + (k0 + 8 * g + (j >> 2)) * pitch + c0 + 4 * (j & 3);
    const s16x4g u0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g_p)(a));
    const s16x4g u1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g_p)(a + 4 * pitch));
    const s16x8g u = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
    return __builtin_bit_cast(bf16x8, u);
}

__device__ inline f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// gen_gemm_nt for bf16 inputs: M[i][j] = alpha sum_c A[i][c] B[j][c], A = Q
// (exact) or dO (split), B = K or V (exact).  d staged 64 columns at a time;
// pitch 72 halves (the 8-lane groups of a 16-byte read start on distinct
// 4-bank groups).
template <int D, int SRCA>
__global__ void __launch_bounds__(NTH) gen_gemm_nt16(GParams p, const void *a_tensor, const void *b_tensor,
                                                     float *slot, float alpha)
{
    typedef typename std::conditional<SRCA == SRC_OBUF, float, bf16_t>::type AT;
    constexpr int NPA = SRCA == SRC_OBUF ? 3 : 1;
    constexpr int KC = D < 64 ? D : 64;
    constexpr int P = KC + 8;
    __shared__ __align__(16) bf16_t As[NPA * TB * P];
    __shared__ __align__(16) bf16_t Bs[TB * P];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB, j0 = jt * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const AT *asrc = static_cast<const AT *>(rows_base<bf16_t, SRCA>(p, a_tensor, x, y));
    const bf16_t *bsrc = static_cast<const bf16_t *>(rows_base<bf16_t, SRC_TENSOR>(p, b_tensor, x, y));
    const int wr = (w >> 1) * 32, wc = (w & 1) * 32;
    const int lr = lane & 15, lk = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < D; c0 += KC) {
        if (c0) __syncthreads();
        stage_rows16<NPA, AT, D, KC>(As, P, asrc, i0, p.T, tid, c0);
        stage_rows16<1, bf16_t, D, KC>(Bs, P, bsrc, j0, p.T, tid, c0);
        __syncthreads();
#pragma unroll
        for (int k0 = 0; k0 < KC; k0 += 32) {
            bf16x8 bv[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                bv[nb] = *reinterpret_cast<const bf16x8 *>(Bs + (wc + 16 * nb + lr) * P + k0 + 8 * lk);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int pl = 0; pl < NPA; ++pl) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(As + pl * TB * P + (wr + 16 * mb + lr) * P + k0 + 8 * lk);
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma16(a, bv[nb], acc[mb][nb]);
                }
        }
    }
    float *m = map_of(slot, p, y);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + wr + 16 * mb + 4 * lk + r, j = j0 + wc + 16 * nb + lr;
                m[(size_t)i * p.Tp + j] = alpha * acc[mb][nb][r];
            }
}

// gen_gemm_mn for bf16 inputs: Out[i][:] = alpha sum_j M[i][j] B[j][:], the
// map split into three planes (pitch 72 halves), B = V or K (exact, pitch
// D + 16 halves: the four rows of a transposing read start 8 banks apart).
template <int D, bool TO_OBUF>
__global__ void __launch_bounds__(NTH) gen_gemm_mn16(GParams p, const float *slot, const void *b_tensor, float *out,
                                                     float alpha)
{
    constexpr int MP = TB + 8, BP = D + 16;
    __shared__ __align__(16) bf16_t Ms[3 * TB * MP];
    __shared__ __align__(16) bf16_t Bs[TB * BP];
    const int it = p.nt - 1 - (int)blockIdx.x, y = blockIdx.y;  // the longest rows first
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const float *m = map_of(const_cast<float *>(slot), p, y);
    const bf16_t *bsrc = static_cast<const bf16_t *>(b_tensor) + tensor_off(p, x);
    f32x4 acc[D / 16];
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int jt_end = it + 1 < p.nt ? it + 1 : p.nt - 1;
    TileRegs mr;
    RowRegs<bf16_t, D> br;
    mr.load(m, p.Tp, i0, 0, tid);
    br.load(bsrc, 0, p.T, tid);
    for (int jt = 0; jt <= jt_end; ++jt) {
        store_tile16<3>(mr, Ms, MP, tid);
        store_rows16<1>(br, Bs, BP, tid);
        __syncthreads();
        if (jt < jt_end) {  // the next tile's reads overlap this tile's products
            mr.load(m, p.Tp, i0, (jt + 1) * TB, tid);
            br.load(bsrc, (jt + 1) * TB, p.T, tid);
        }
#pragma unroll
        for (int k0 = 0; k0 < TB; k0 += 32) {
            bf16x8 a[3];
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
                a[pl] = *reinterpret_cast<const bf16x8 *>(Ms + pl * TB * MP + (16 * w + lr) * MP + k0 + 8 * lk);
#pragma unroll
            for (int n = 0; n < D / 16; ++n) {
                const bf16x8 b = tr_frag(Bs, BP, k0, 16 * n, lane);
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) acc[n] = mfma16(a[pl], b, acc[n]);
            }
        }
        __syncthreads();
    }
    float *o = TO_OBUF ? p.obuf + (size_t)y * p.T * D : out + tensor_off(p, x);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 16 * w + 4 * lk + r;
            if (i < p.T) o[(size_t)i * D + 16 * n + lr] = alpha * acc[n][r];
        }
}

// gen_gemm_tn for bf16 inputs with an exact B (dK = dS^T Q): Out[j][:] =
// alpha sum_i M[i][j] B[i][:], both operands read along the rows i with
// transposing reads (map planes: pitch 72 halves, the four rows of a read 36
// banks apart mod 64).
template <int D>
__global__ void __launch_bounds__(NTH) gen_gemm_tn16(GParams p, const float *slot, const void *b_tensor, float *out,
                                                     float alpha)
{
    constexpr int MP = TB + 8, BP = D + 16;
    __shared__ __align__(16) bf16_t Ms[3 * TB * MP];
    __shared__ __align__(16) bf16_t Bs[TB * BP];
    const int jt = blockIdx.x, y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int j0 = jt * TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const float *m = map_of(const_cast<float *>(slot), p, y);
    const bf16_t *bsrc = static_cast<const bf16_t *>(b_tensor) + tensor_off(p, x);
    f32x4 acc[D / 16];
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int it0 = jt > 0 ? jt - 1 : 0;
    TileRegs mr;
    RowRegs<bf16_t, D> br;
    mr.load(m, p.Tp, it0 * TB, j0, tid);
    br.load(bsrc, it0 * TB, p.T, tid);
    for (int it = it0; it < p.nt; ++it) {
        store_tile16<3>(mr, Ms, MP, tid);
        store_rows16<1>(br, Bs, BP, tid);
        __syncthreads();
        if (it + 1 < p.nt) {  // the next tile's reads overlap this tile's products
            mr.load(m, p.Tp, (it + 1) * TB, j0, tid);
            br.load(bsrc, (it + 1) * TB, p.T, tid);
        }
#pragma unroll
        for (int k0 = 0; k0 < TB; k0 += 32) {
            bf16x8 a[3];
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) a[pl] = tr_frag(Ms + pl * TB * MP, MP, k0, 16 * w, lane);
#pragma unroll
            for (int n = 0; n < D / 16; ++n) {
                const bf16x8 b = tr_frag(Bs, BP, k0, 16 * n, lane);
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) acc[n] = mfma16(a[pl], b, acc[n]);
            }
        }
        __syncthreads();
    }
    float *o = out + tensor_off(p, x);
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + 16 * w + 4 * lk + r;
            if (j < p.T) o[(size_t)j * D + 16 * n + lr] = alpha * acc[n][r];
        }
}

// ---------------------------------------------------------------------------
// Stencils (fp32 VALU).  A thread owns 16 consecutive columns of one row of a
// 64 x 64 output tile; for each kernel row it loads a window of 16 + c_k - 1
// input values into registers and walks the taps with register indices.

// Stages rows r0 .. r0 + nr - 1, columns c0 .. c0 + XP - 1 of a map into LDS
// (pitch XP): map[r][c] where 0 <= r < T, c < c0 + ncol and 0 <= c <= r +
// cadd, else zero.  25 float4 per row, 10 rows per pass (threads 250..255
// idle); no barrier inside.
__device__ inline void stage_region(float *dst, const float *m, const GParams &p, int r0, int c0, int nr,
                                    int ncol, int cadd, int tid)
{
    static_assert(XP == 100, "25 float4 per row");
    if (tid >= 250) return;
    const int c4 = tid % 25, rsub = tid / 25;
    for (int rr = rsub; rr < nr; rr += 10) {
        const int r = r0 + rr;
        const bool rok = r >= 0 && r < p.T;
        const float *row = m + (size_t)(rok ? r : 0) * p.Tp;
        const int cmax = min(p.T - 1, r + cadd);
        float4 v;
        float *vv = reinterpret_cast<float *>(&v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = 4 * c4 + e, c = c0 + cc;
            vv[e] = (rok && cc < ncol && c >= 0 && c <= cmax) ? row[c] : 0.f;
        }
        *reinterpret_cast<float4 *>(dst + rr * XP + 4 * c4) = v;
    }
}

// Input region of the forward stencil and of the kernel gradient: rows
// i0 - (c_q - 1) .. i0 + 63, columns j0 - hi .. j0 + 63 - lo (hi = c_k - 1 -
// floor(c_k/2), lo = -floor(c_k/2)), with the mode's masks:
//   M_PRE  : Mask_0 (column <= row), M_POST: probabilities, zero past the
//   diagonal; M_EXACT: the raw map up to c_q - 1 past the diagonal (Eq. 4's
//   indicator is applied per tap by the caller).
template <int MODE>
__device__ inline void stage_input(float *Xs, const float *m, const GParams &p, int i0, int j0, int tid)
{
    const int hi = p.c_k - 1 - p.c_k / 2;
    stage_region(Xs, m, p, i0 - (p.c_q - 1), j0 - hi, TB + p.c_q - 1, TB + p.c_k - 1,
                 MODE == M_EXACT ? p.c_q - 1 : 0, tid);
}

// Loads the register window win[x] = row[16 q + x] of an LDS region row.
// (16-byte reads through a native vector type, so that they stay ds_read_b128)
__device__ inline void load_win(float (&win)[WIN], const float *row)
{
#pragma unroll
    for (int x = 0; x < WIN; x += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(row + x);
        win[x] = t[0];
        win[x + 1] = t[1];
        win[x + 2] = t[2];
        win[x + 3] = t[3];
    }
}

// out = Eq. 4 on the input map (mode's masks), then Mask_0, on every band
// tile (grid: n_band x heads).
// Dynamic LDS of the stencil kernels: `regions` input regions of
// (64 + c_q - 1) x XP floats, then the kernel taps (and their gradient).
inline size_t conv_lds_bytes(int c_q, int regions)
{
    return ((size_t)regions * (TB + c_q - 1) * XP + 2 * MAX_CQ * 32) * sizeof(float);
}

template <int MODE>
__global__ void __launch_bounds__(NTH) gen_conv_fwd(GParams p, const float *in_slot, float *out_slot)
{
    extern __shared__ __align__(16) float lds_dyn[];
    float *Xs = lds_dyn;
    float *th = Xs + (TB + p.c_q - 1) * XP;
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB, j0 = jt * TB;
    const int tid = threadIdx.x;
    const int rl = tid >> 2, q = tid & 3;
    const int i = i0 + rl;
    float *out = map_of(out_slot, p, y);
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    if (jt <= it) {  // the tile right of the diagonal is zero after Mask_0
        stage_input<MODE>(Xs, map_of(const_cast<float *>(in_slot), p, y), p, i0, j0, tid);
        for (int t = tid; t < p.c_q * p.c_k; t += NTH) th[t] = p.theta[(size_t)x.h * p.c_q * p.c_k + t];
        __syncthreads();
        const int hi = p.c_k - 1 - p.c_k / 2;
        for (int ip = 0; ip < p.c_q; ++ip) {
            float win[WIN];
            load_win(win, Xs + (rl - ip + p.c_q - 1) * XP + 16 * q);
            if (MODE == M_EXACT) {  // Eq. 4's indicator: the input key must not pass the output row
#pragma unroll
                for (int xx = 0; xx < WIN; ++xx)
                    if (j0 - hi + 16 * q + xx > i) win[xx] = 0.f;
            }
            const float *tr = th + ip * p.c_k;
#pragma unroll
            for (int s = 0; s < 31; ++s) {
                if (s < p.c_k) {
                    const float t = tr[p.c_k - 1 - s];
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[e] = fmaf(t, win[e + s], acc[e]);
                }
            }
        }
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        float4 v;
        float *vv = reinterpret_cast<float *>(&v);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = j0 + 16 * q + 4 * e4 + c;
            vv[c] = (i < p.T && j <= i) ? acc[4 * e4 + c] : 0.f;
        }
        *reinterpret_cast<float4 *>(out + (size_t)i * p.Tp + j0 + 16 * q + 4 * e4) = v;
    }
}

// The convolution's backward on every band tile (grid: n_band x heads), with
// G = Mask_0 of the gradient at the convolution's output (column <= row):
//   dIn[r][c] = sum_taps theta[i'][j'] G[r + i'][c + j']  (M_PRE: for c <= r;
//               M_EXACT: each tap only where c <= r + i', Eq. 4's indicator;
//               M_POST: for c <= r, where the probabilities are not zero)
//   dtheta[h][i'][j'] += sum over the tile's G[i][j] x input[i - i'][j - j']
//               (the input with the mode's masks, as in the forward).
template <int MODE>
__global__ void __launch_bounds__(NTH) gen_conv_bwd(GParams p, const float *g_slot, const float *in_slot,
                                                    float *din_slot)
{
    extern __shared__ __align__(16) float lds_dyn[];
    float *Gs = lds_dyn;
    float *Xs = Gs + (TB + p.c_q - 1) * XP;
    float *th = Xs + (TB + p.c_q - 1) * XP;
    float *dth = th + MAX_CQ * 32;
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int i0 = it * TB, j0 = jt * TB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int rl = tid >> 2, q = tid & 3;
    const int r = i0 + rl;
    const int lo = -(p.c_k / 2), hi = p.c_k - 1 - p.c_k / 2;
    const bool upper = jt > it;
    float *din = map_of(din_slot, p, y);
    if (upper && MODE != M_EXACT) {  // nothing reaches past the diagonal tile
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            *reinterpret_cast<float4 *>(din + (size_t)r * p.Tp + j0 + 16 * q + 4 * e4) =
                make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    const float *gm = map_of(const_cast<float *>(g_slot), p, y);
    // G region: rows i0 .. i0 + 63 + c_q - 1, columns j0 + lo .. (Mask_0 applied)
    stage_region(Gs, gm, p, i0, j0 + lo, TB + p.c_q - 1, TB + p.c_k - 1, 0, tid);
    if (!upper) stage_input<MODE>(Xs, map_of(const_cast<float *>(in_slot), p, y), p, i0, j0, tid);
    for (int t = tid; t < p.c_q * p.c_k; t += NTH) {
        th[t] = p.theta[(size_t)x.h * p.c_q * p.c_k + t];
        dth[t] = 0.f;
    }
    __syncthreads();

    // dIn
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int ip = 0; ip < p.c_q; ++ip) {
        float win[WIN];
        load_win(win, Gs + (rl + ip) * XP + 16 * q);
        const float *tr = th + ip * p.c_k;
        float tmp[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) tmp[e] = 0.f;
#pragma unroll
        for (int s = 0; s < 31; ++s) {
            if (s < p.c_k) {
                const float t = tr[s];
#pragma unroll
                for (int e = 0; e < 16; ++e) tmp[e] = fmaf(t, win[e + s], tmp[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (MODE == M_EXACT)
                acc[e] += (j0 + 16 * q + e <= r + ip) ? tmp[e] : 0.f;
            else
                acc[e] += tmp[e];
        }
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        float4 v;
        float *vv = reinterpret_cast<float *>(&v);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int cj = j0 + 16 * q + 4 * e4 + c;
            const int cmax = MODE == M_EXACT ? r + p.c_q - 1 : r;
            vv[c] = (r < p.T && cj < p.T && cj <= cmax) ? acc[4 * e4 + c] : 0.f;
        }
        *reinterpret_cast<float4 *>(din + (size_t)r * p.Tp + j0 + 16 * q + 4 * e4) = v;
    }
    if (upper) return;  // no G element of the tile right of the diagonal survives Mask_0

    // dtheta: this thread's G elements G[r][j0 + 16 q + e] against the input
    // window of each kernel row, reduced over the wave 16 taps at a time.
    float g[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) g[e] = Gs[rl * XP + 16 * q + e - lo];
    for (int ip = 0; ip < p.c_q; ++ip) {
        float win[WIN];
        load_win(win, Xs + (rl - ip + p.c_q - 1) * XP + 16 * q);
        if (MODE == M_EXACT) {
#pragma unroll
            for (int xx = 0; xx < WIN; ++xx)
                if (j0 - hi + 16 * q + xx > r) win[xx] = 0.f;
        }
#pragma unroll
        for (int s0 = 0; s0 < 32; s0 += 16) {
            if (s0 < p.c_k) {
                float part[16];
#pragma unroll
                for (int ss = 0; ss < 16; ++ss) {
                    float sacc = 0.f;
                    if (s0 + ss < p.c_k) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) sacc = fmaf(g[e], win[e + s0 + ss], sacc);
                    }
                    part[ss] = sacc;
                }
                const float tot = reduce16(part, lane);
                const int s = s0 + reduce16_slot(lane);
                if ((lane & 3) == 0 && s < p.c_k) atomicAdd(&dth[ip * p.c_k + (p.c_k - 1 - s)], tot);
            }
        }
    }
    __syncthreads();
    for (int t = tid; t < p.c_q * p.c_k; t += NTH) atomicAdd(p.dtheta + (size_t)x.h * p.c_q * p.c_k + t, dth[t]);
}

// ---------------------------------------------------------------------------
// Row kernels: one wave per row of a head's map (grid: Tp / 4 x heads).

// In place: L -> P = softmax over the row's causal entries (Mask_-inf), zero
// past the diagonal up to the end of the row's band tiles.
__global__ void __launch_bounds__(NTH) gen_softmax_fwd(GParams p, float *slot)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    float *row = map_of(slot, p, blockIdx.y) + (size_t)i * p.Tp;
    const int band_end = min(p.Tp, (i / TB + 2) * TB);
    const int n = i < p.T ? i + 1 : 0;
    float m = -INFINITY, l = 0.f;
    for (int j = 4 * lane; j < n; j += 256) {
        const float4 v = load4(row + j);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (j + c < n) {
                const float xv = vv[c];
                if (xv > m) {
                    l = l * __expf(m - xv) + 1.0f;
                    m = xv;
                } else {
                    l += __expf(xv - m);
                }
            }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float mo = __shfl_xor(m, o), lo_ = __shfl_xor(l, o);
        const float mn = fmaxf(m, mo);
        l = (m == -INFINITY ? 0.f : l * __expf(m - mn)) + (mo == -INFINITY ? 0.f : lo_ * __expf(mo - mn));
        m = mn;
    }
    const float il = l > 0.f ? 1.0f / l : 0.f;
    for (int j = 4 * lane; j < band_end; j += 256) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < n) v = load4(row + j);
        float *vv = reinterpret_cast<float *>(&v);
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = (j + c < n) ? __expf(vv[c] - m) * il : 0.f;
        *reinterpret_cast<float4 *>(row + j) = v;
    }
}

// In place in the gradient slot: dP -> dL = P (dP - sum_j P dP), zero past the
// diagonal.
__global__ void __launch_bounds__(NTH) gen_softmax_bwd(GParams p, const float *p_slot, float *g_slot)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const float *prow = map_of(const_cast<float *>(p_slot), p, blockIdx.y) + (size_t)i * p.Tp;
    float *grow = map_of(g_slot, p, blockIdx.y) + (size_t)i * p.Tp;
    const int band_end = min(p.Tp, (i / TB + 2) * TB);
    const int n = i < p.T ? i + 1 : 0;
    float dsum = 0.f;
    for (int j = 4 * lane; j < n; j += 256) {
        const float4 a = load4(prow + j), b = load4(grow + j);
        const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (j + c < n) dsum = fmaf(av[c], bv[c], dsum);
    }
    dsum = wave_sum(dsum);
    for (int j = 4 * lane; j < band_end; j += 256) {
        float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < n) {
            const float4 a = load4(prow + j), b = load4(grow + j);
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
            float *ov = reinterpret_cast<float *>(&out);
#pragma unroll
            for (int c = 0; c < 4; ++c) ov[c] = (j + c < n) ? av[c] * (bv[c] - dsum) : 0.f;
        }
        *reinterpret_cast<float4 *>(grow + j) = out;
    }
}

// ---------------------------------------------------------------------------
// Head mixes within a group (Eq. 7), elementwise over the band tiles of the
// group's c_h heads (grid: n_band x units of the chunk).  CH = c_h.

// out^a = sum_b w[g][a][b] in^b (in place allowed).
template <int CH>
__global__ void __launch_bounds__(NTH) gen_mix_fwd(GParams p, const float *in_slot, float *out_slot)
{
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int uu = blockIdx.y, g = (p.u0 + uu) % p.G;
    float w[CH][CH];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int b = 0; b < CH; ++b) w[a][b] = p.w[((size_t)g * CH + a) * CH + b];
    const size_t msz = (size_t)p.Tp * p.Tp;
    const float *in = in_slot + (size_t)uu * CH * msz;
    float *out = out_slot + (size_t)uu * CH * msz;
    for (int idx = threadIdx.x; idx < TB * TB / 4; idx += NTH) {
        const int rr = idx >> 4, c4 = idx & 15;
        const size_t off = (size_t)(it * TB + rr) * p.Tp + jt * TB + 4 * c4;
        float4 v[CH];
#pragma unroll
        for (int b = 0; b < CH; ++b) v[b] = load4(in + b * msz + off);
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int b = 0; b < CH; ++b) {
                o.x = fmaf(w[a][b], v[b].x, o.x);
                o.y = fmaf(w[a][b], v[b].y, o.y);
                o.z = fmaf(w[a][b], v[b].z, o.z);
                o.w = fmaf(w[a][b], v[b].w, o.w);
            }
            *reinterpret_cast<float4 *>(out + a * msz + off) = o;
        }
    }
}

// In place in the gradient slot: dOut -> dIn^b = sum_a w_ab dOut^a, and
// dw[g][a][b] += sum over causal entries of dOut^a x in^b (in: the mix's
// forward input).
template <int CH>
__global__ void __launch_bounds__(NTH) gen_mix_bwd(GParams p, float *g_slot, const float *in_slot)
{
    __shared__ float dws[16];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int uu = blockIdx.y, g = (p.u0 + uu) % p.G;
    const int tid = threadIdx.x, lane = tid & 63;
    float w[CH][CH];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int b = 0; b < CH; ++b) w[a][b] = p.w[((size_t)g * CH + a) * CH + b];
    if (tid < 16) dws[tid] = 0.f;
    const size_t msz = (size_t)p.Tp * p.Tp;
    float *gm = g_slot + (size_t)uu * CH * msz;
    const float *in = in_slot + (size_t)uu * CH * msz;
    float part[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) part[t] = 0.f;
    for (int idx = tid; idx < TB * TB / 4; idx += NTH) {
        const int rr = idx >> 4, c4 = idx & 15;
        const int i = it * TB + rr, j = jt * TB + 4 * c4;
        const size_t off = (size_t)i * p.Tp + j;
        float4 go[CH], xi[CH];
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            go[a] = load4(gm + a * msz + off);
            xi[a] = load4(in + a * msz + off);
        }
        float mk[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) mk[c] = (i < p.T && j + c <= i) ? 1.f : 0.f;
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int b = 0; b < CH; ++b) {
                const float s = mk[0] * go[a].x * xi[b].x + mk[1] * go[a].y * xi[b].y + mk[2] * go[a].z * xi[b].z +
                                mk[3] * go[a].w * xi[b].w;
                part[a * CH + b] += s;
            }
#pragma unroll
        for (int b = 0; b < CH; ++b) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                o.x = fmaf(w[a][b], go[a].x, o.x);
                o.y = fmaf(w[a][b], go[a].y, o.y);
                o.z = fmaf(w[a][b], go[a].z, o.z);
                o.w = fmaf(w[a][b], go[a].w, o.w);
            }
            *reinterpret_cast<float4 *>(gm + b * msz + off) = o;
        }
    }
    __syncthreads();
    const float tot = reduce16(part, lane);
    const int slot = reduce16_slot(lane);
    if ((lane & 3) == 0 && slot < CH * CH) atomicAdd(&dws[slot], tot);
    __syncthreads();
    if (tid < CH * CH) atomicAdd(p.dw + (size_t)g * CH * CH + tid, dws[tid]);
}

// Groups of 8 or 16 heads: the same mixes with the group's weights in LDS
// (c_h^2 of them would not fit the registers), and the dw sums in a kernel
// of their own, one output head a per grid z, run before the gradient is
// transformed in place.
template <int CH>
__global__ void __launch_bounds__(NTH) gen_mix_fwd_wide(GParams p, const float *in_slot, float *out_slot)
{
    __shared__ float ws[CH * CH];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int uu = blockIdx.y, g = (p.u0 + uu) % p.G;
    for (int t = threadIdx.x; t < CH * CH; t += NTH) ws[t] = p.w[(size_t)g * CH * CH + t];
    __syncthreads();
    const size_t msz = (size_t)p.Tp * p.Tp;
    const float *in = in_slot + (size_t)uu * CH * msz;
    float *out = out_slot + (size_t)uu * CH * msz;
    for (int idx = threadIdx.x; idx < TB * TB / 4; idx += NTH) {
        const int rr = idx >> 4, c4 = idx & 15;
        const size_t off = (size_t)(it * TB + rr) * p.Tp + jt * TB + 4 * c4;
        float4 v[CH];
#pragma unroll
        for (int b = 0; b < CH; ++b) v[b] = load4(in + b * msz + off);
#pragma unroll 2
        for (int a = 0; a < CH; ++a) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int b = 0; b < CH; ++b) {
                const float wab = ws[a * CH + b];
                o.x = fmaf(wab, v[b].x, o.x);
                o.y = fmaf(wab, v[b].y, o.y);
                o.z = fmaf(wab, v[b].z, o.z);
                o.w = fmaf(wab, v[b].w, o.w);
            }
            *reinterpret_cast<float4 *>(out + a * msz + off) = o;
        }
    }
}

// dw[g][a][b] += sum over causal entries of dOut^a x in^b, a = blockIdx.z
// (grid: n_band x units of the chunk x c_h).
template <int CH>
__global__ void __launch_bounds__(NTH) gen_mix_dw_wide(GParams p, const float *g_slot, const float *in_slot)
{
    static_assert(CH <= 16, "one partial per source head and lane group");
    __shared__ float dws[16];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int uu = blockIdx.y, g = (p.u0 + uu) % p.G, a = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 16) dws[tid] = 0.f;
    const size_t msz = (size_t)p.Tp * p.Tp;
    const float *gm = g_slot + ((size_t)uu * CH + a) * msz;
    const float *in = in_slot + (size_t)uu * CH * msz;
    float part[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) part[t] = 0.f;
    for (int idx = tid; idx < TB * TB / 4; idx += NTH) {
        const int rr = idx >> 4, c4 = idx & 15;
        const int i = it * TB + rr, j = jt * TB + 4 * c4;
        const size_t off = (size_t)i * p.Tp + j;
        float4 go = load4(gm + off);
        const bool row_in = i < p.T;
        go.x = (row_in && j <= i) ? go.x : 0.f;
        go.y = (row_in && j + 1 <= i) ? go.y : 0.f;
        go.z = (row_in && j + 2 <= i) ? go.z : 0.f;
        go.w = (row_in && j + 3 <= i) ? go.w : 0.f;
#pragma unroll
        for (int b = 0; b < CH; ++b) {
            const float4 xi = load4(in + b * msz + off);
            part[b] += go.x * xi.x + go.y * xi.y + go.z * xi.z + go.w * xi.w;
        }
    }
    __syncthreads();
    const float tot = reduce16(part, lane);
    const int slot = reduce16_slot(lane);
    if ((lane & 3) == 0 && slot < CH) atomicAdd(&dws[slot], tot);
    __syncthreads();
    if (tid < CH) atomicAdd(p.dw + ((size_t)g * CH + a) * CH + tid, dws[tid]);
}

// In place in the gradient slot: dOut -> dIn^b = sum_a w_ab dOut^a.
template <int CH>
__global__ void __launch_bounds__(NTH) gen_mix_bwd_wide(GParams p, float *g_slot)
{
    __shared__ float ws[CH * CH];
    int it, jt;
    band_tile(blockIdx.x, p.nt, it, jt);
    const int uu = blockIdx.y, g = (p.u0 + uu) % p.G;
    for (int t = threadIdx.x; t < CH * CH; t += NTH) ws[t] = p.w[(size_t)g * CH * CH + t];
    __syncthreads();
    const size_t msz = (size_t)p.Tp * p.Tp;
    float *gm = g_slot + (size_t)uu * CH * msz;
    for (int idx = threadIdx.x; idx < TB * TB / 4; idx += NTH) {
        const int rr = idx >> 4, c4 = idx & 15;
        const size_t off = (size_t)(it * TB + rr) * p.Tp + jt * TB + 4 * c4;
        float4 go[CH];
#pragma unroll
        for (int a = 0; a < CH; ++a) go[a] = load4(gm + a * msz + off);
#pragma unroll 2
        for (int b = 0; b < CH; ++b) {
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                const float wab = ws[a * CH + b];
                o.x = fmaf(wab, go[a].x, o.x);
                o.y = fmaf(wab, go[a].y, o.y);
                o.z = fmaf(wab, go[a].z, o.z);
                o.w = fmaf(wab, go[a].w, o.w);
            }
            *reinterpret_cast<float4 *>(gm + b * msz + off) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// GroupNorm backward, one wave per token of one head (grid: ceil(T / 64) x
// heads; each workgroup 64 tokens).  In place in the O buffer: O -> dO.
template <typename DT, int D>
__global__ void __launch_bounds__(NTH) gen_groupnorm_bwd(GParams p)
{
    constexpr int NCH = D >= 64 ? D / 64 : 1;  // channels per lane
    __shared__ float red[4][2 * D + 1];
    const int y = blockIdx.y;
    const HeadIx x = head_ix(p, y);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool on = D >= 64 || lane < D;
    const float sig = p.gate ? 1.0f / (1.0f + __expf(-p.gate[x.h])) : 1.0f;
    const float scale = p.depth_scale * sig;
    float gam[NCH], bet[NCH], dgam[NCH], dbet[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int ch = lane + 64 * c;
        gam[c] = on ? p.gn_w[(size_t)x.h * D + ch] : 0.f;
        bet[c] = on ? p.gn_b[(size_t)x.h * D + ch] : 0.f;
        dgam[c] = dbet[c] = 0.f;
    }
    float dg = 0.f;
    float *o = p.obuf + (size_t)y * p.T * D;
    const DT *dy = static_cast<const DT *>(p.dout) + tensor_off(p, x);
    const float inv_d = 1.0f / (float)D;
    for (int t = blockIdx.x * 64 + w; t < min(p.T, (int)(blockIdx.x + 1) * 64); t += 4) {
        float ov[NCH], gv[NCH];
        float s1 = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            ov[c] = on ? o[(size_t)t * D + ch] : 0.f;
            gv[c] = on ? to_f(dy[(size_t)t * D + ch]) : 0.f;
            s1 += ov[c];
        }
        const float mu = wave_sum(s1) * inv_d;
        float s2 = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float dd = on ? ov[c] - mu : 0.f;
            s2 += dd * dd;
        }
        const float var = wave_sum(s2) * inv_d;
        const float rstd = 1.0f / sqrtf(var + p.eps);
        float xh[NCH], dxh[NCH];
        float sa = 0.f, sb = 0.f, sg = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            xh[c] = on ? (ov[c] - mu) * rstd : 0.f;
            dxh[c] = scale * gam[c] * gv[c];
            sa += dxh[c];
            sb += dxh[c] * xh[c];
            sg += gv[c] * (gam[c] * xh[c] + bet[c]);
            dgam[c] = fmaf(scale * gv[c], xh[c], dgam[c]);
            dbet[c] += scale * gv[c];
        }
        const float ma = wave_sum(sa) * inv_d, mb = wave_sum(sb) * inv_d;
        dg += wave_sum(sg);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = lane + 64 * c;
            if (on) o[(size_t)t * D + ch] = rstd * (dxh[c] - ma - xh[c] * mb);
        }
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (on) {
            red[w][lane + 64 * c] = dgam[c];
            red[w][D + lane + 64 * c] = dbet[c];
        }
    if (lane == 0) red[w][2 * D] = dg;
    __syncthreads();
    for (int t = tid; t < 2 * D + 1; t += NTH) {
        const float s = red[0][t] + red[1][t] + red[2][t] + red[3][t];
        if (t < D)
            atomicAdd(p.dgn_w + (size_t)x.h * D + t, s);
        else if (t < 2 * D)
            atomicAdd(p.dgn_b + (size_t)x.h * D + (t - D), s);
        else if (p.gate)  // d/dg of depth_scale * sigmoid(g) * z = depth_scale * sig (1 - sig) * z
            atomicAdd(p.dgate + x.h, s * p.depth_scale * sig * (1.0f - sig));
    }
}

}  // namespace gen
}  // namespace mta
