// mta_bwd.h — gradients of the MTA forward on gfx950 for the default placement:
// key-query convolution before the softmax (two-pass masks, or Eq. 4's exact
// indicator), head mixing after it (Eq. 7), GroupNorm x depth scale (x optional
// sigmoid gate) (page "Multi-Token Attention — Paper Graph", section 3.4).
//
// Forward, per head (log2-domain quantities as in the forward kernels):
//   S = Q K^T / sqrt(d);  X = Mask_0(S) (two-pass) or S (exact);
//   C = Conv2d_theta(X);  P = softmax(Mask_-inf(C));  P3^a = sum_b w_ab P^b;
//   O^a = P3^a V^a;  Y^a = (GN(O^a) * gamma + beta) * s_a.
// Backward, given dY:
//   dO^a from the GroupNorm backward; dV^a = P3^aT dO^a; dP3^a = dO^a V^aT;
//   dP^b = sum_a w_ab dP3^a;  dw_ab = sum dP3^a . P^b;
//   dC^b = P^b (dP^b - D^b),  D^b_i = sum_j P^b_ij dP^b_ij = sum_a w_ab dO^a_i . (P^b V^a)_i;
//   dX^b = Conv2d^T_theta(dC^b);  dtheta^b = corr(dC^b, X^b);  dS = Mask_0(dX) (or dX);
//   dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
//
// Kernel A (one workgroup per (b, head group, 64 query rows), 4 waves): the
// forward again (statistics pass, then probabilities), accumulating P^b V^a for
// every (source, output) head pair; the epilogue forms O, the GroupNorm
// backward (dO, atomics into dgamma, dbeta, dgate) and D^b, and writes the row
// statistics, D and dO (in the input dtype) to the workspace.
//
// Kernel B (one workgroup per (b, head group, 64-key tile), 4 waves) walks the
// query tiles that reach its keys.  Per query tile it recomputes, on a region
// extended by the convolution's reach (rows below and keys on both sides of
// the tile, since the transposed convolution reads dC there), the logits X,
// the convolved map and P, and dP3 on the matrix cores; forms dC in LDS;
// accumulates dtheta (LDS atomics), dw, dV and dK (registers), computes dS with
// the transposed stencil and adds dS K into dQ with global atomics.
#pragma once

#include "mta_fwd_layer.h"

namespace mta {
namespace bwd {

constexpr int NT = 256;         // kernel A: 4 waves
constexpr int NTB = 512;        // kernel B: 8 waves, two per SIMD
constexpr int NWB = NTB / 64;

typedef _Float16 h16_t;
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
// fp16 copy of the logit region for the matrix-core stencil: halves per row
constexpr int X16P = 104;
// bf16 copy of the dC core for the matrix-core kernel gradient (in the fp16
// logit copy's space, free by then): 72 halves per row, so that the 16 rows a
// fragment read touches start on distinct 4-bank groups
constexpr int DCP = 72;

// Kernels with compile-time stencil sizes (bf16, d = 128) recompute the
// convolved map on the matrix cores, as the head-split forward does: fp16
// operands (the logit region and the banded kernel matrices), fp32 sums.
template <typename DT, int D, int CQ, int CK>
constexpr bool stencil_on_mfma() { return sizeof(DT) == 2 && D == 128 && CQ > 0 && CK > 0 && CK <= 17; }

// bytes of the fp16 logit region and of both heads' banded kernel matrices
// (0 for the kernels that keep the VALU stencil)
__host__ __device__ constexpr int ms_bytes(bool on, int nrrb, int ch, int cq)
{
    return on ? nrrb * 16 * X16P * 2 + ch * cq * 64 * 16 : 0;
}

struct BParams {
    Params f;                        // forward geometry and pointers (q, k, v, theta, wmix, gn, gate)
    const void *dout;                // dY [B][H][T][d] (input dtype)
    float *dq, *dk, *dv;             // [B][H][T][d] fp32
    float *dtheta, *dw, *dgn_w, *dgn_b, *dgate;
    float *ws_m, *ws_il, *ws_D;      // workspace: row statistics (log2 max, 1/sum) and D, [B][H][T]
    void *ws_dO;                     // workspace: dO [B][H][T][d] in the input dtype (bf16: the high part)
    void *ws_dOl;                    // workspace, bf16 only: dO - high part, in bf16
    // kernel B geometry
    int hr;                          // floor(c_k/2)
    int nEr, nEc, epitch;            // extended dC region: rows, columns, floats per row
    int nRrb, nRcb, xpitch;          // logit region: 16-row / 16-column blocks, floats per row
    float inv_sqrt_d, inv_log2e;
};

// Buffers cleared before the kernels accumulate into them.
struct ZeroList {
    float *p[6];
    size_t n[6];
    int k;
};

typedef hipError_t (*BwdFn)(const BParams &p, int grid_a, size_t lds_a, int grid_b, size_t lds_b, hipStream_t s);

// ---------------------------------------------------------------------------
// P.V-shaped product with an fp32 A operand (lane: one row, 16 k values).  With
// bf16 operands the A values are split into bf16 hi + lo and both are
// multiplied (the B operand is exact input data), so the product keeps about
// 16 significant bits of A; fp32 runs one fp32 product.
template <int D>
__device__ inline void pv_x(f32x4 (&acc)[D / 16], const float a[16], const bf16_t *buf, int lane)
{
    float hi[16], lo[16];
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        hi[o] = (float)(bf16_t)a[o];
        lo[o] = a[o] - hi[o];
    }
    pv_mfma<D>(acc, hi, buf, lane);
    pv_mfma<D>(acc, lo, buf, lane);
}
template <int D>
__device__ inline void pv_x(f32x4 (&acc)[D / 16], const float a[16], const float *buf, int lane)
{
    pv_mfma<D>(acc, a, buf, lane);
}

// The same products for half of the d-columns: 16-column blocks
// [nb0, nb0 + D/32) of the B operand (layout of load_v_tile / TileStage).
template <int D>
__device__ inline void pv_half(f32x4 (&acc)[D / 32], const float pr[16], const bf16_t *vb, int lane, int nb0)
{
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (bf16_t)pr[8 * c + e];
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            const bf16x8 bv =
                *reinterpret_cast<const bf16x8 *>(vb + ((nb0 + nb) * 16 + n) * VP_BF16 + kg * 16 + 8 * c);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[nb], 0, 0, 0);
        }
    }
}
template <int D>
__device__ inline void pv_half(f32x4 (&acc)[D / 32], const float pr[16], const float *vb, int lane, int nb0)
{
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            const float bv = vb[(kg * 16 + t) * (D + 4) + (nb0 + nb) * 16 + n];
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[t], bv, acc[nb], 0, 0, 0);
        }
    }
}
template <int D>
__device__ inline void pv_x_half(f32x4 (&acc)[D / 32], const float a[16], const bf16_t *buf, int lane, int nb0)
{
    float hi[16], lo[16];
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        hi[o] = (float)(bf16_t)a[o];
        lo[o] = a[o] - hi[o];
    }
    pv_half<D>(acc, hi, buf, lane, nb0);
    pv_half<D>(acc, lo, buf, lane, nb0);
}
template <int D>
__device__ inline void pv_x_half(f32x4 (&acc)[D / 32], const float a[16], const float *buf, int lane, int nb0)
{
    pv_half<D>(acc, a, buf, lane, nb0);
}

// ---------------------------------------------------------------------------
// Kernel A
template <typename DT, int D, int CH, int CQ, int CK>
__global__ void __launch_bounds__(NT) mta_bwd_prep(BParams bp)
{
    const Params &p = bp.f;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;
    const int cq = CQ ? CQ : p.c_q;
    const int ck = CK ? CK : p.c_k;
    const int ckp = (ck + 3) & ~3;

    float *sbuf = lds;
    float *th_s = sbuf + EXT_R * p.pitch;                 // [CH][cq][ckp]
    float *w_s = th_s + ((CH * cq * ckp + 3) & ~3);       // [CH][CH]
    float *red = w_s + ((CH * CH + 3) & ~3);              // [4 waves][CH][2][D] partial GN sums
    float *gred = red + 4 * CH * 2 * D;                   // [4 waves][CH] gate partials
    DT *vbuf = reinterpret_cast<DT *>(gred + ((4 * CH + 3) & ~3));

    const size_t hstride = (size_t)T * D;
    const DT *Q = reinterpret_cast<const DT *>(p.q);
    const DT *K = reinterpret_cast<const DT *>(p.k);
    const DT *V = reinterpret_cast<const DT *>(p.v);
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;

    for (int i = tid; i < CH * cq * ckp; i += NT) {
        const int a = i / (cq * ckp), r = (i / ckp) % cq, c = i % ckp;
        th_s[i] = c < ck ? p.theta[((size_t)(h0 + a) * cq + r) * ck + c] : 0.f;
    }
    for (int i = tid; i < CH * CH; i += NT) w_s[i] = p.wmix[(size_t)g * CH * CH + i];

    const int io = wave * 16 + (lane & 15);
    const int jb = 16 * (lane >> 4);
    const int qabs = i0 + io;
    const int rho = HALO + io;

    // pass 1: statistics of the convolved logits
    float m_c[CH], l_c[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        m_c[a] = NEG_INF;
        l_c[a] = 0.f;
    }
    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        const int tlim = p.exact ? qabs - (j0 - p.hl + jb) : (1 << 30);
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            float c[16];
            __syncthreads();
            logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride, i0, j0, nullptr,
                                   nullptr, wave, lane);
            __syncthreads();
            stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + a * cq * ckp, cq, ck, ckp, tlim, c);
            stats_update(c, j0 + jb, qabs, m_c[a], l_c[a]);
        }
    }
    float M[CH], IL[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) stats_merge(m_c[a], l_c[a], M[a], IL[a]);
    if (lane < 16 && qabs < T) {
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            const size_t ri = ((size_t)b * p.H + h0 + a) * T + qabs;
            bp.ws_m[ri] = M[a];
            bp.ws_il[ri] = IL[a];
        }
    }

    // pass 2: U[s][a] = P^s V^a for every pair
    f32x4 U[CH][CH][D / 16];
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) U[s][a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        const int tlim = p.exact ? qabs - (j0 - p.hl + jb) : (1 << 30);
        float pr[CH][16];
#pragma unroll
        for (int s = 0; s < CH; ++s) {
            __syncthreads();
            logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + s * hstride, K + base0 + s * hstride, i0, j0, nullptr,
                                   nullptr, wave, lane);
            __syncthreads();
            stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + s * cq * ckp, cq, ck, ckp, tlim, pr[s]);
#pragma unroll
            for (int o = 0; o < 16; ++o)
                pr[s][o] = (j0 + jb + o <= qabs) ? __builtin_amdgcn_exp2f(pr[s][o] - M[s]) * IL[s] : 0.f;
        }
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            __syncthreads();
            load_v_tile<D>(vbuf, V + base0 + a * hstride, j0, T, tid);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < CH; ++s) pv_x<D>(U[s][a], pr[s], vbuf, lane);
        }
    }

    // epilogue: O, GroupNorm backward, D.  Lane: rows 16*wave + 4*(lane/16) + r,
    // columns 16*nb + lane%16.
    const DT *dY = reinterpret_cast<const DT *>(bp.dout);
    DT *dO_ws = reinterpret_cast<DT *>(bp.ws_dO);
    DT *dOl_ws = reinterpret_cast<DT *>(bp.ws_dOl);
    const int n = lane & 15;
    float dOr[CH][D / 16][4];
    float gpart[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        const int h = h0 + a;
        const float *gw = p.gn_w + (size_t)h * D;
        const float *gb = p.gn_b + (size_t)h * D;
        const float sg = p.gate ? 1.0f / (1.0f + __expf(-p.gate[h])) : 1.0f;
        const float sa = p.depth_scale * sg;
        float dgw[D / 16], dgb[D / 16];
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) dgw[nb] = dgb[nb] = 0.f;
        gpart[a] = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = i0 + wave * 16 + 4 * (lane >> 4) + r;
            const bool live = row < T;
            float x[D / 16];
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                float o = 0.f;
#pragma unroll
                for (int s = 0; s < CH; ++s) o = __builtin_fmaf(w_s[a * CH + s], U[s][a][nb][r], o);
                x[nb] = o;
            }
            float sum = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) sum += x[nb];
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            sum += __shfl_xor(sum, 8);
            const float mu = sum * (1.0f / D);
            float v2 = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const float dl = x[nb] - mu;
                v2 = __builtin_fmaf(dl, dl, v2);
            }
            v2 += __shfl_xor(v2, 1);
            v2 += __shfl_xor(v2, 2);
            v2 += __shfl_xor(v2, 4);
            v2 += __shfl_xor(v2, 8);
            const float rstd = 1.0f / __builtin_sqrtf(v2 * (1.0f / D) + p.eps);
            float xh[D / 16], dxh[D / 16];
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const int col = 16 * nb + n;
                xh[nb] = (x[nb] - mu) * rstd;
                const float dy = live ? (float)dY[((size_t)b * p.H + h) * hstride + (size_t)row * D + col] : 0.f;
                const float dys = dy * sa;
                dgb[nb] += dys;
                dgw[nb] = __builtin_fmaf(dys, xh[nb], dgw[nb]);
                gpart[a] = __builtin_fmaf(dy, xh[nb] * gw[col] + gb[col], gpart[a]);
                dxh[nb] = dys * gw[col];
                s1 += dxh[nb];
                s2 = __builtin_fmaf(dxh[nb], xh[nb], s2);
            }
            s1 += __shfl_xor(s1, 1);
            s1 += __shfl_xor(s1, 2);
            s1 += __shfl_xor(s1, 4);
            s1 += __shfl_xor(s1, 8);
            s2 += __shfl_xor(s2, 1);
            s2 += __shfl_xor(s2, 2);
            s2 += __shfl_xor(s2, 4);
            s2 += __shfl_xor(s2, 8);
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const float dox = rstd * (dxh[nb] - s1 * (1.0f / D) - xh[nb] * s2 * (1.0f / D));
                // stored as the input dtype, with the bf16 remainder in a second plane
                const DT dh = cvt_out<DT>(dox);
                if (live) {
                    const size_t at = ((size_t)b * p.H + h) * hstride + (size_t)row * D + 16 * nb + n;
                    dO_ws[at] = dh;
                    if (sizeof(DT) == 2) dOl_ws[at] = cvt_out<DT>(dox - (float)dh);
                }
                dOr[a][nb][r] = live ? dox : 0.f;
            }
        }
        // dgamma, dbeta: the four lane groups of a column, then the waves via LDS
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
            float u = dgw[nb], t = dgb[nb];
            u += __shfl_xor(u, 16);
            u += __shfl_xor(u, 32);
            t += __shfl_xor(t, 16);
            t += __shfl_xor(t, 32);
            if (lane < 16) {
                red[((wave * CH + a) * 2 + 0) * D + 16 * nb + n] = u;
                red[((wave * CH + a) * 2 + 1) * D + 16 * nb + n] = t;
            }
        }
        float gsum = gpart[a];
#pragma unroll
        for (int sh = 1; sh < 64; sh <<= 1) gsum += __shfl_xor(gsum, sh);
        if (lane == 0) gred[wave * CH + a] = gsum * p.depth_scale * sg * (1.0f - sg);
    }
    __syncthreads();
    for (int i = tid; i < CH * 2 * D; i += NT) {
        const int a = i / (2 * D), which = (i / D) % 2, col = i % D;
        float t = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) t += red[((w4 * CH + a) * 2 + which) * D + col];
        atomicAdd((which ? bp.dgn_b : bp.dgn_w) + (size_t)(h0 + a) * D + col, t);
    }
    if (p.gate && tid < CH) {
        float t = 0.f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) t += gred[w4 * CH + tid];
        atomicAdd(bp.dgate + h0 + tid, t);
    }
    // D^s_i = sum_a w_as dO^a_i . (P^s V^a)_i
#pragma unroll
    for (int s = 0; s < CH; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float t = 0.f;
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                float u = 0.f;
#pragma unroll
                for (int nb = 0; nb < D / 16; ++nb) u = __builtin_fmaf(dOr[a][nb][r], U[s][a][nb][r], u);
                t = __builtin_fmaf(w_s[a * CH + s], u, t);
            }
            t += __shfl_xor(t, 1);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 4);
            t += __shfl_xor(t, 8);
            const int row = i0 + wave * 16 + 4 * (lane >> 4) + r;
            if (n == 0 && row < T) bp.ws_D[((size_t)b * p.H + h0 + s) * T + row] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel B helpers

// Transposed key-query stencil: 16 outputs of one row of dX,
//   dX[r][c] = sum_{i'} sum_{jj} theta[i'][jj] dC[r + i'][c + jj - floor(c_k/2)],
// from the extended dC region (its row er + i' holds dC row r + i', its column
// jb + o + jj holds key c + jj - floor(c_k/2) for output column c = j0 + jb + o).
// With Eq. 4's indicator the terms of query offset i' count only where
// c <= r + i', i.e. o <= dlim + i' with dlim = r - j0 - jb.
// Only the query offsets i' = ip0, ip0 + 2, ... are summed (the two waves that
// share a row split them).
template <int CQ, int CK>
__device__ inline void stencil16_t(const float *ebuf, int pitch, int er, int jb, const float *th, int cq_rt,
                                   int ck_rt, int ckp, int dlim, int ip0, float out[16])
{
    constexpr int MAXW = CK ? 16 + CK - 1 : 16 + MAX_CK - 1;
    constexpr int MAXW4 = (MAXW + 3) / 4;
    constexpr int KMAX = CK ? CK : MAX_CK;
    const int cq = CQ ? CQ : cq_rt;
    const int ck = CK ? CK : ck_rt;
    const int nw4 = (16 + ck - 1 + 3) / 4;
#pragma unroll
    for (int o = 0; o < 16; ++o) out[o] = 0.f;
    for (int ip = ip0; ip < cq; ip += 2) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(ebuf + (er + ip) * pitch + jb);
        float win[MAXW4 * 4];
#pragma unroll
        for (int t = 0; t < MAXW4; ++t) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (CK || t < nw4) x = row[t];
            win[4 * t + 0] = x[0];
            win[4 * t + 1] = x[1];
            win[4 * t + 2] = x[2];
            win[4 * t + 3] = x[3];
        }
        const float *trow = th + ip * ckp;
        float tmp[16];
#pragma unroll
        for (int o = 0; o < 16; ++o) tmp[o] = 0.f;
#pragma unroll
        for (int jj = 0; jj < KMAX; ++jj) {
            if (CK || jj < ck) {
                const float tv = trow[jj];
#pragma unroll
                for (int o = 0; o < 16; ++o) tmp[o] = __builtin_fmaf(tv, win[o + jj], tmp[o]);
            }
        }
#pragma unroll
        for (int o = 0; o < 16; ++o) out[o] += (o <= dlim + ip) ? tmp[o] : 0.f;
    }
}

// Sum of x over the 64 lanes of the wave, in every lane: rotations by 8, 4, 2, 1
// within each 16-lane row (DPP row_ror), then the rows pairwise
// (v_permlane16_swap, v_permlane32_swap).
__device__ inline float wave_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(x);
    const auto b2 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(b2[0]) + __uint_as_float(b2[1]);
}

// dtheta[i'][jj] += sum_o g[o] * X[row - i'][col(o) + floor(c_k/2) - jj] for the
// lane's 16 values g (one row, 16 keys); each tap's sum over the wave is added
// into LDS by one lane (atomics between the waves).  The
// logit region's row rx0 holds the lane's row minus 0 offsets: window of query
// offset i' starts at row rx0 - i', column xc0 (the key col(0) - (c_k - 1) +
// floor(c_k/2)); window entries t > tlim are keys in the future of the row
// (Eq. 4's indicator) and are skipped.  Only the query offsets i' = ip0,
// ip0 + 2, ... are done (the two waves that share a row split them).
template <int CQ, int CK>
__device__ inline void dtheta16(const float *xbuf, int pitch, int rx0, int xc0, const float g[16], float *dth,
                                int cq_rt, int ck_rt, int ckp, int tlim, int ip0)
{
    constexpr int MAXW = CK ? 16 + CK - 1 : 16 + MAX_CK - 1;
    constexpr int MAXW4 = (MAXW + 3) / 4;
    constexpr int KMAX = CK ? CK : MAX_CK;
    const int cq = CQ ? CQ : cq_rt;
    const int ck = CK ? CK : ck_rt;
    const int nw = 16 + ck - 1;
    const int nw4 = (nw + 3) / 4;
    for (int ip = ip0; ip < cq; ip += 2) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(xbuf + (rx0 - ip) * pitch + xc0);
        float win[MAXW4 * 4];
#pragma unroll
        for (int t = 0; t < MAXW4; ++t) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (CK || t < nw4) x = row[t];
            win[4 * t + 0] = x[0];
            win[4 * t + 1] = x[1];
            win[4 * t + 2] = x[2];
            win[4 * t + 3] = x[3];
        }
        if (tlim < nw - 1) {
#pragma unroll
            for (int t = 0; t < MAXW; ++t) win[t] = (t <= tlim) ? win[t] : 0.f;
        }
        // tap jj reads window entry o + c_k - 1 - jj; with m = c_k - 1 - jj the
        // register index o + m is static.  The taps are independent
        // accumulators; after the wave sums lane m holds tap m and one LDS
        // atomic instruction adds them all.
        float acc[KMAX];
#pragma unroll
        for (int m = 0; m < KMAX; ++m) acc[m] = 0.f;
#pragma unroll
        for (int o = 0; o < 16; ++o)
#pragma unroll
            for (int m = 0; m < KMAX; ++m)
                if (CK || m < ck) acc[m] = __builtin_fmaf(g[o], win[o + m], acc[m]);
        const int lane = threadIdx.x & 63;
        float v = 0.f;
#pragma unroll
        for (int m = 0; m < KMAX; ++m)
            if (CK || m < ck) {
                const float t = wave_sum(acc[m]);
                v = (lane == m) ? t : v;
            }
        if (lane < ck) atomicAdd(dth + ip * ckp + (ck - 1 - lane), v);
    }
}

// dtheta on the matrix cores (bf16 operands, fp32 sums; two-pass masks):
//   dtheta[i'][jj] = sum over the core (r, c) of dC[r][c] X[r - i'][c + hr - jj]
//                  = sum over logit rows r' and core keys c of A[jj][c] B[c][i'],
//   A[jj][c] = X[r'][c + hr - jj] (a Toeplitz band of one logit row),
//   B[c][i'] = dC[r' + i'][c]     (c_q consecutive dC rows),
// one 16x16x32 product per (logit row, 32-key chunk), the tasks dealt to the
// waves; each wave adds its sums (lane: tap 4*(lane/16) + q, query offset
// lane%16) into dth [c_q][ckp] with LDS atomics.  xbuf: the fp32 logit region
// (row r' + c_q - 1, column c + hr + c_k - 1 - jj for key c of the core); dcb:
// the bf16 dC core.
template <int CQ, int CK>
__device__ inline void dtheta_mfma(float *dth, int ckp, const float *xbuf, int xp, const bf16_t *dcb, int hr,
                                   int wave, int lane)
{
    const int m = lane & 15, g = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int t = wave; t < 2 * (BM + CQ - 1); t += NWB) {
        const int xr = t >> 1, c0 = 32 * (t & 1);
        const int rd = xr - (CQ - 1) + m;  // the dC row of this lane's B column (query offset m)
        bf16x8 a, bv;
        if (m < CK) {
            float xv[8];
            __builtin_memcpy(xv, xbuf + xr * xp + c0 + 8 * g + hr + CK - 1 - m, sizeof(xv));
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (bf16_t)xv[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (bf16_t)0.0f;
        }
        if (m < CQ && rd >= 0 && rd < BM) {
            bv = *reinterpret_cast<const bf16x8 *>(dcb + rd * DCP + c0 + 8 * g);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = (bf16_t)0.0f;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc, 0, 0, 0);
    }
    if (m < CQ) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (4 * g + q < CK) atomicAdd(dth + m * ckp + 4 * g + q, acc[q]);
    }
}

// The nrb x ncb 16x16 blocks of a region product, in row-major order, are dealt
// to the NWB waves in contiguous runs; a run loads the row fragments again
// where its row block changes and requests the next column fragments before
// each product.  f(rb, cb, acc) stores one block (lane: row lane%16, columns
// 4*(lane/16) .. +3).
// A row fragment as load_frag, addressed as the wave-uniform head base plus a
// 32-bit lane offset (row < T <= 2^24, so row * D * sizeof(DT) < 2^32 at d =
// 128 in bf16 and at d <= 64 in float32): the compiler can keep the base in
// scalar registers and use the scalar-base form of the load, one VGPR per
// fragment stream instead of a 64-bit address.  Held as 64-bit addresses
// across the query-tile loop they were spilled, and each reload waited for
// every global load in flight.
template <int D>
__device__ inline void load_frag_s(QFrag<D> &f, const bf16_t *base, int row, int T, int lane)
{
    const unsigned off = (unsigned)row * (unsigned)(D * 2) + (unsigned)((lane >> 4) * (D / 4) * 2);
    if ((unsigned)row < (unsigned)T) {
        const bf16x8 *p = reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(base) + off);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) f.x[t] = p[t];
    } else {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) f.x[t][e] = (bf16_t)0.0f;
    }
}
template <int D>
__device__ inline void load_frag_s(QFrag32<D> &f, const float *base, int row, int T, int lane)
{
    load_frag<D>(f, base, row, T, lane);
}

template <typename DT, int D, bool SPLIT, typename F>
__device__ inline void region_product(int nrb, int ncb, const DT *rh, const DT *rl, int r0, const DT *ch, int c0,
                                      int T, int wave, int lane, F &&f)
{
    typedef typename FragOf<DT, D>::type Frag;
    const int n = nrb * ncb, t0 = wave * n / NWB, t1 = (wave + 1) * n / NWB;
    if (t0 >= t1) return;
    Frag hf, lf, cf, cn;
    int rcur = -1;
    load_frag_s<D>(cf, ch, c0 + 16 * (t0 % ncb) + (lane & 15), T, lane);
    for (int t = t0; t < t1; ++t) {
        const int rb = t / ncb, cb = t % ncb;
        if (rb != rcur) {
            const int qi = r0 + 16 * rb + (lane & 15);
            load_frag_s<D>(hf, rh, qi, T, lane);
            if (SPLIT) load_frag_s<D>(lf, rl, qi, T, lane);
            rcur = rb;
        }
        if (t + 1 < t1) load_frag_s<D>(cn, ch, c0 + 16 * ((t + 1) % ncb) + (lane & 15), T, lane);
        f32x4 acc = qk_mfma<D>(cf, hf);
        if (SPLIT) {
            const f32x4 a2 = qk_mfma<D>(cf, lf);
            acc += a2;
        }
        cf = cn;
        f(rb, cb, acc);
    }
}

// dP3 tile: buf[row][col] = dO[r0 + row] . V[c0 + col] over rows < nrows (0
// outside [0, T)); with SPLIT the product of the low plane of dO is added.
template <typename DT, int D, bool SPLIT>
__device__ inline void prod_tile(float *buf, int pitch, int nrb, int ncb, int nrows, const DT *dh, const DT *dl,
                                 const DT *vh, int r0, int c0, int T, int wave, int lane)
{
    region_product<DT, D, SPLIT>(nrb, ncb, dh, dl, r0, vh, c0, T, wave, lane, [&](int rb, int cb, const f32x4 &acc) {
        if (16 * rb + (lane & 15) < nrows)
            *reinterpret_cast<f32x4 *>(buf + (16 * rb + (lane & 15)) * pitch + 16 * cb + 4 * (lane >> 4)) = acc;
    });
}

// Logit region X: buf[row][col] = sc * Q[r0 + row] . K[c0 + col], 0 outside
// [0, T) and, unless raw, where the key is in the future of the row (Mask_0).
// With x16, the same values also go to an fp16 copy (pitch X16P).
template <typename DT, int D>
__device__ inline void x_tile(float *buf, int pitch, int nrb, int ncb, int nrows, const DT *qh, const DT *kh, int r0,
                              int c0, int T, float sc, bool raw, int wave, int lane, h16_t *x16 = nullptr)
{
    region_product<DT, D, false>(nrb, ncb, qh, qh, r0, kh, c0, T, wave, lane, [&](int rb, int cb, const f32x4 &acc) {
        const int qi = r0 + 16 * rb + (lane & 15);
        const int e0 = 16 * cb + 4 * (lane >> 4);
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kj = c0 + e0 + r;
            const bool ok = qi >= 0 && qi < T && kj >= 0 && kj < T && (raw || kj <= qi);
            o[r] = ok ? acc[r] * sc : 0.f;
        }
        if (16 * rb + (lane & 15) < nrows) *reinterpret_cast<f32x4 *>(buf + (16 * rb + (lane & 15)) * pitch + e0) = o;
        if (x16) {
            const h16x4 h = {(h16_t)o[0], (h16_t)o[1], (h16_t)o[2], (h16_t)o[3]};
            *reinterpret_cast<h16x4 *>(x16 + (16 * rb + (lane & 15)) * X16P + e0) = h;
        }
    });
}

// A 64-row tile for the P.V-shaped products of kernel B (layout of
// load_v_tile), staged in registers: fetch() issues the global loads, put()
// writes the LDS tile, so that a tile's loads can be in flight while the
// previous tile is used.
template <typename DT, int D>
struct TileStage;

template <int D>
struct TileStage<bf16_t, D> {
    // thread -> key tid % 64 and the 8-channel chunks tid / 64 + NWB * it
    static constexpr int NC = D / 8, IT = (NC + NWB - 1) / NWB;
    bf16x8 x[IT];
    __device__ void fetch(const bf16_t *g, int r0, int T, int tid)
    {
        const int key = tid & 63, kj = r0 + key;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int ch = (tid >> 6) + NWB * it;
            if (ch < NC && kj < T) {
                // wave-uniform head base + 32-bit lane offset (as load_frag_s)
                const unsigned off = (unsigned)kj * (unsigned)(D * 2) + 16u * (unsigned)ch;
                x[it] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(g) + off);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[it][e] = (bf16_t)0.0f;
            }
        }
    }
    __device__ void put(bf16_t *vb, int tid) const
    {
        const int key = tid & 63;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int ch = (tid >> 6) + NWB * it;
            if (ch < NC) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vb[(8 * ch + e) * VP_BF16 + key] = x[it][e];
            }
        }
    }
};

template <int D>
struct TileStage<float, D> {
    static constexpr int C4 = D / 4, N = BN * C4 / NTB;
    f32x4 x[N];
    __device__ void fetch(const float *g, int r0, int T, int tid)
    {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = tid + it * NTB, key = idx / C4, c0 = (idx % C4) * 4, kj = r0 + key;
            x[it] = kj < T ? *reinterpret_cast<const f32x4 *>(g + (size_t)kj * D + c0) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ void put(float *vb, int tid) const
    {
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int idx = tid + it * NTB, key = idx / C4, c0 = (idx % C4) * 4;
            *reinterpret_cast<f32x4 *>(vb + key * (D + 4) + c0) = x[it];
        }
    }
};

// ---------------------------------------------------------------------------
// Kernel B
// EXM: 0 = the masking form from p.exact (runtime); 1 = two-pass masks, 2 =
// Eq. 4's indicator, fixed at compile time (the kernels with compile-time
// stencils, which then carry only one form's code)
template <typename DT, int D, int CH, int CQ, int CK, int EXM = 0>
__global__ void __launch_bounds__(NTB) mta_bwd_main(BParams bp)
{
    const Params &p = bp.f;
    const bool exact = EXM == 0 ? p.exact != 0 : EXM == 2;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int kt = L / p.units;  // workgroups with the most query tiles first
    const int b = unit / p.G, g = unit % p.G;
    const int j0 = kt * BN;
    const int T = p.T;
    const int cq = CQ ? CQ : p.c_q;
    const int ck = CK ? CK : p.c_k;
    const int ckp = (ck + 3) & ~3;
    const int hr = bp.hr, hl = p.hl;
    const int nEr = bp.nEr, nEc = bp.nEc, ep = bp.epitch, xp = bp.xpitch;

    // LDS carve-up
    float *xbuf = lds;                                            // logits X / later dS core
    float *ebuf = xbuf + bp.nRrb * 16 * xp;                       // C -> P -> dC (extended region)
    float *dpb = ebuf + nEr * ep;                                 // dP3^a, [CH][nEr][ep]
    float *th_s = dpb + CH * nEr * ep;                            // [CH][cq][ckp]
    float *w_s = th_s + ((CH * cq * ckp + 3) & ~3);
    float *dth = w_s + ((CH * CH + 3) & ~3);                      // accumulated dtheta [CH][cq][ckp]
    float *st = dth + ((CH * cq * ckp + 3) & ~3);                 // [CH][3][nEr4]: m, il, D of the region rows
    const int nEr4 = (nEr + 3) & ~3;
    float *dwr = st + CH * 3 * nEr4;                              // [NWB waves][CH*CH]
    DT *opbuf = reinterpret_cast<DT *>(dwr + ((NWB * CH * CH + 3) & ~3));
    constexpr bool MS = stencil_on_mfma<DT, D, CQ, CK>();
    // MS: fp16 copy of the logit region, then both heads' banded kernel matrices
    h16_t *x16 = reinterpret_cast<h16_t *>(reinterpret_cast<char *>(opbuf) + vbuf_bytes<DT, D>());
    h16x8 *tfl = reinterpret_cast<h16x8 *>(x16 + bp.nRrb * 16 * X16P);  // [s][i'][lane]
    // MS: the bf16 dC core for the kernel gradient on the matrix cores, in the
    // fp16 logit copy's space (free once the convolved map of the head is
    // formed); with Eq. 4's indicator only for query tiles two or more below
    // the key tile, where every tap's key lies in the past of every output row
    // (key <= j0 + 63 + hr < i0), so the indicator passes all of them
    bf16_t *dcb = reinterpret_cast<bf16_t *>(x16);

    const size_t hstride = (size_t)T * D;
    const DT *Q = reinterpret_cast<const DT *>(p.q);
    const DT *K = reinterpret_cast<const DT *>(p.k);
    const DT *V = reinterpret_cast<const DT *>(p.v);
    const DT *dO = reinterpret_cast<const DT *>(bp.ws_dO);
    const DT *dOl = reinterpret_cast<const DT *>(bp.ws_dOl);
    constexpr bool SPLIT = sizeof(DT) == 2;  // bf16: dO carried as hi + lo planes
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;

    for (int i = tid; i < CH * cq * ckp; i += NTB) {
        const int a = i / (cq * ckp), r = (i / ckp) % cq, c = i % ckp;
        th_s[i] = c < ck ? p.theta[((size_t)(h0 + a) * cq + r) * ck + c] : 0.f;
    }
    for (int i = tid; i < CH * cq * ckp; i += NTB) dth[i] = 0.f;
    for (int i = tid; i < CH * CH; i += NTB) w_s[i] = p.wmix[(size_t)g * CH * CH + i];
    if constexpr (MS) {
        // banded kernel matrices (MFMA A operands): lane row m = lane%16 (output
        // key), columns k = 8*(lane/16) + e of the 32-column window, tap
        // j' = m + c_k - 1 - k
        __syncthreads();
        for (int i = tid; i < CH * CQ * 64; i += NTB) {
            const int sh = i / (CQ * 64), ip = (i / 64) % CQ, ln = i % 64;
            h16x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = (ln & 15) + CK - 1 - (8 * (ln >> 4) + e);
                f[e] = (h16_t)((jj >= 0 && jj < CK) ? th_s[(sh * CQ + ip) * ckp + jj] : 0.f);
            }
            tfl[i] = f;
        }
    }
    float dwp[CH * CH];
#pragma unroll
    for (int i = 0; i < CH * CH; ++i) dwp[i] = 0.f;


    // waves w and w + 4 share rows / keys: they split the query offsets of the
    // stencils and the d-columns of the products (half = w / 4)
    const int wq = wave & 3, half = wave >> 2;
    const int nb0 = half * (D / 32);       // first 16-column block of the wave's d-half
    const int io = wq * 16 + (lane & 15);  // the lane's row (stencil layout) within a query tile
    const int jb = 16 * (lane >> 4);       // its first key within the key tile
    const int km = wq * 16 + (lane & 15);  // its key (transposed operand layout)
    const int rk = 16 * (lane >> 4);       // its first row (transposed operand layout)

    f32x4 dK[CH][D / 32], dV[CH][D / 32];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            dK[a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            dV[a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int nlcb = (nEc + 15) / 16;
    const int qt0 = exact ? (kt > 0 ? kt - 1 : 0) : kt;
    // The 64-row tiles of one (query tile, head s) step, in order of use:
    // dO^a (and its low plane) for every output head a, K^s at the key tile,
    // Q^s at the query tile.  Each is fetched into registers one tile ahead.
    constexpr int NDO = SPLIT ? 2 * CH : CH;
    TileStage<DT, D> stg;
    auto fetch_tile = [&](int qt, int s, int k) {
        if (qt >= p.n_qt) return;
        if (k < NDO) {
            const int a = SPLIT ? k >> 1 : k;
            const DT *src = (SPLIT && (k & 1)) ? dOl : dO;
            stg.fetch(src + base0 + a * hstride, qt * BM, T, tid);
        } else if (k == NDO) {
            stg.fetch(K + base0 + s * hstride, j0, T, tid);
        } else {
            stg.fetch(Q + base0 + s * hstride, qt * BM, T, tid);
        }
    };
    // put tile k of step (qt, s) into LDS, then request the one after it
    auto put_tile = [&](int qt, int s, int k) {
        stg.put(opbuf, tid);
        if (k + 1 <= NDO + 1) fetch_tile(qt, s, k + 1);
        else if (s + 1 < CH) fetch_tile(qt, s + 1, 0);
        else fetch_tile(qt + 1, 0, 0);
    };
    fetch_tile(qt0, 0, 0);
    for (int qt = qt0; qt < p.n_qt; ++qt) {
        const int i0 = qt * BM;
        const bool grad_mfma = MS && (!exact || qt >= kt + 2);
        const int ec0 = j0 - hr;              // key of region column 0
        const int xr0 = i0 - (cq - 1);        // query of logit row 0
        const int xc0 = ec0 - hl;             // key of logit column 0
        __syncthreads();
        // row statistics and D of the region's rows
        for (int i = tid; i < CH * nEr; i += NTB) {
            const int a = i / nEr, r = i % nEr;
            const int row = i0 + r;
            const size_t ri = ((size_t)b * p.H + h0 + a) * T + row;
            const bool live = row < T;
            st[(a * 3 + 0) * nEr4 + r] = live ? bp.ws_m[ri] : 0.f;
            st[(a * 3 + 1) * nEr4 + r] = live ? bp.ws_il[ri] : 0.f;
            st[(a * 3 + 2) * nEr4 + r] = live ? bp.ws_D[ri] : 0.f;
        }
        // dP3^a over the region: dO^a rows x V^a keys (no scale, no mask; bf16:
        // high and low planes of dO)
        for (int a = 0; a < CH; ++a)
            prod_tile<DT, D, SPLIT>(dpb + a * nEr * ep, ep, (nEr + 15) / 16, nlcb, nEr, dO + base0 + a * hstride,
                                    dOl + base0 + a * hstride, V + base0 + a * hstride, i0, ec0, T, wave, lane);

#pragma unroll
        for (int s = 0; s < CH; ++s) {
            __syncthreads();
            // X^s over the logit region (log2-scaled; Mask_0 unless exact)
            x_tile<DT, D>(xbuf, xp, bp.nRrb, bp.nRcb, 16 * bp.nRrb, Q + base0 + s * hstride, K + base0 + s * hstride,
                          xr0, xc0, T, p.sc, exact, wave, lane, (MS && !exact) ? x16 : nullptr);
            __syncthreads();
            // C^s over the region -> P^s (in place)
            if (MS && !exact) {
                // on the matrix cores (two-pass masks; Eq. 4's indicator keeps the
                // VALU stencil): 16x16 blocks (region rows 16rb.., columns 16cb..)
                // dealt to the waves; lane: row 16rb + lane%16, columns 16cb + 4*(lane/16) + r
                // The centre tap is exact: the accumulators start from
                // theta_00 x - fp16(theta_00) fp16(x) at the output positions (x
                // from the fp32 region), as the forward that produced the
                // statistics makes it exact.
                const h16x8 *tfs = tfl + s * CQ * 64;
                const float t00 = th_s[s * cq * ckp + CK / 2], t00h = (float)(h16_t)t00;
                const int nrb = (nEr + 15) / 16, nxr = 16 * bp.nRrb;
                for (int tsk = wave; tsk < nrb * nlcb; tsk += NWB) {
                    const int rb = tsk / nlcb, cb = tsk % nlcb;
                    const int r = 16 * rb + (lane & 15);
                    f32x4 acc;
                    {
                        int xr = r + CQ - 1;
                        xr = xr < nxr ? xr : nxr - 1;  // rows past the region: results unused
                        const int xc = 16 * cb + 4 * (lane >> 4) + p.hl;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[q] = __builtin_fmaf(t00, xbuf[xr * xp + xc + q], -t00h * (float)x16[xr * X16P + xc + q]);
                    }
#pragma unroll
                    for (int ip = 0; ip < CQ; ++ip) {
                        int xr = r + CQ - 1 - ip;
                        xr = xr < nxr ? xr : nxr - 1;  // rows past the region: results unused
                        const h16x8 xv = *reinterpret_cast<const h16x8 *>(x16 + xr * X16P + 16 * cb + 8 * (lane >> 4));
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(tfs[ip * 64 + lane], xv, acc, 0, 0, 0);
                    }
                    if (r < nEr) {
                        const int qi = i0 + r;
                        const float m = st[(s * 3 + 0) * nEr4 + r], il = st[(s * 3 + 1) * nEr4 + r];
                        f32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int kj = ec0 + 16 * cb + 4 * (lane >> 4) + q;
                            o[q] = (kj >= 0 && kj <= qi && qi < T) ? __builtin_amdgcn_exp2f(acc[q] - m) * il : 0.f;
                        }
                        *reinterpret_cast<f32x4 *>(ebuf + r * ep + 16 * cb + 4 * (lane >> 4)) = o;
                    }
                }
            } else
            for (int t = tid; t < nEr * nlcb; t += NTB) {
                const int r = t / nlcb, cb = t % nlcb;
                const int qi = i0 + r;
                const int tlim = exact ? qi - (xc0 + 16 * cb) : (1 << 30);
                float o[16];
                stencil16<CQ, CK>(xbuf, xp, r + cq - 1, 16 * cb, th_s + s * cq * ckp, cq, ck, ckp, tlim, o);
                const float m = st[(s * 3 + 0) * nEr4 + r], il = st[(s * 3 + 1) * nEr4 + r];
                float *dst = ebuf + r * ep + 16 * cb;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kj = ec0 + 16 * cb + e;
                    dst[e] = (kj >= 0 && kj <= qi && qi < T) ? __builtin_amdgcn_exp2f(o[e] - m) * il : 0.f;
                }
            }
            __syncthreads();
            // dV^a += w_as P^sT dO^a (core rows i0.., keys j0..): split P against
            // dO's high plane, P's high part against dO's low plane
            for (int a = 0; a < CH; ++a) {
                __syncthreads();
                put_tile(qt, s, SPLIT ? 2 * a : a);
                __syncthreads();
                float at[16];
                const float wa = w_s[a * CH + s];
#pragma unroll
                for (int o = 0; o < 16; ++o) at[o] = wa * ebuf[(rk + o) * ep + hr + km];
                pv_x_half<D>(dV[a], at, opbuf, lane, nb0);
                if (SPLIT) {
                    __syncthreads();
                    put_tile(qt, s, 2 * a + 1);
                    __syncthreads();
                    float ah[16];
#pragma unroll
                    for (int o = 0; o < 16; ++o) ah[o] = (float)(bf16_t)at[o];
                    pv_half<D>(dV[a], ah, opbuf, lane, nb0);
                }
            }
            __syncthreads();
            // dC^s = P^s (sum_a w_as dP3^a - D^s) in place; dw partials over the core
            for (int idx = tid; idx < nEr * nEc; idx += NTB) {
                const int r = idx / nEc, c = idx % nEc;
                const float pv = ebuf[r * ep + c];
                float dp = 0.f;
                const bool core = r < BM && c >= hr && c < hr + BN;
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    const float x = dpb[(a * nEr + r) * ep + c];
                    dp = __builtin_fmaf(w_s[a * CH + s], x, dp);
                    if (core) dwp[a * CH + s] = __builtin_fmaf(x, pv, dwp[a * CH + s]);
                }
                const float dcv = pv * (dp - st[(s * 3 + 2) * nEr4 + r]);
                ebuf[r * ep + c] = dcv;
                if (grad_mfma && core) dcb[r * DCP + c - hr] = (bf16_t)dcv;
            }
            __syncthreads();
            // dtheta^s += corr(dC core, X^s)
            if (grad_mfma) {
                dtheta_mfma<CQ, CK>(dth + s * cq * ckp, ckp, xbuf, xp, dcb, hr, wave, lane);
            } else {
                float gc[16];
#pragma unroll
                for (int o = 0; o < 16; ++o) gc[o] = ebuf[io * ep + hr + jb + o];
                const int qi = i0 + io;
                // window of the lane: logit row (io + cq-1) - i', columns from jb + hr (key j0 + jb - hl)
                const int tlim = exact ? qi - (xc0 + jb + hr) : (1 << 30);
                dtheta16<CQ, CK>(xbuf, xp, io + cq - 1, jb + hr, gc, dth + s * cq * ckp, cq, ck, ckp, tlim, half);
            }
            // dS^s core = Mask_0(dX) (two-pass) or dX (exact): the transposed stencil,
            // this wave's query offsets; with Eq. 4's indicator the terms of offset
            // i' count where key <= r + i'.  (On the VALU in fp32: dS meets K and
            // Q in products whose rows sum to about zero, which a bf16 dC would
            // not survive.)
            float dsv[16];
            stencil16_t<CQ, CK>(ebuf, ep, io, jb, th_s + s * cq * ckp, cq, ck, ckp,
                                exact ? i0 + io - j0 - jb : (1 << 30), half, dsv);
            __syncthreads();  // xbuf free (dtheta done), ebuf reads done
            // the second half's partial sums meet the first half's in LDS; the
            // first half writes dS core row-major (pitch BN + 4) into xbuf
            float *xch = ebuf + (wq * 64 + lane) * 16;
            if (half) {
#pragma unroll
                for (int o = 0; o < 16; o += 4)
                    *reinterpret_cast<f32x4 *>(xch + o) = f32x4{dsv[o], dsv[o + 1], dsv[o + 2], dsv[o + 3]};
            }
            put_tile(qt, s, NDO);  // K^s
            __syncthreads();
            float *dsb = xbuf;
            if (!half) {
                const int r = i0 + io;
#pragma unroll
                for (int o = 0; o < 16; ++o) {
                    const int c = j0 + jb + o;
                    const bool keep = exact ? true : (c <= r);
                    const float v = dsv[o] + xch[o];
                    dsb[io * (BN + 4) + jb + o] = (keep && r < T && c < T) ? v : 0.f;
                }
            }
            __syncthreads();
            // dQ^s += dS K^s / sqrt(d)  (global atomics; this wave's d-half)
            {
                float at[16];
#pragma unroll
                for (int o = 0; o < 16; ++o) at[o] = dsb[io * (BN + 4) + jb + o];
                f32x4 qa[D / 32];
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb) qa[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
                pv_x_half<D>(qa, at, opbuf, lane, nb0);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int row = i0 + wq * 16 + 4 * (lane >> 4) + r4;
                    if (row < T) {
                        float *dst = bp.dq + ((size_t)b * p.H + h0 + s) * hstride + (size_t)row * D;
#pragma unroll
                        for (int nb = 0; nb < D / 32; ++nb)
                            atomicAdd(dst + 16 * (nb0 + nb) + (lane & 15), qa[nb][r4] * bp.inv_sqrt_d);
                    }
                }
            }
            __syncthreads();  // K^s reads done
            put_tile(qt, s, NDO + 1);  // Q^s
            __syncthreads();
            {
                float at[16];
#pragma unroll
                for (int o = 0; o < 16; ++o) at[o] = dsb[(rk + o) * (BN + 4) + km];
                pv_x_half<D>(dK[s], at, opbuf, lane, nb0);
            }
        }
    }

    // write dK, dV of the key tile; reduce dtheta and dw into the outputs
    for (int a = 0; a < CH; ++a) {
        const size_t hb = ((size_t)b * p.H + h0 + a) * hstride;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int key = j0 + wq * 16 + 4 * (lane >> 4) + r4;
            if (key < T) {
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb) {
                    bp.dk[hb + (size_t)key * D + 16 * (nb0 + nb) + (lane & 15)] = dK[a][nb][r4] * bp.inv_sqrt_d;
                    bp.dv[hb + (size_t)key * D + 16 * (nb0 + nb) + (lane & 15)] = dV[a][nb][r4];
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CH * CH; ++i) {
        float t = dwp[i];
#pragma unroll
        for (int sh = 1; sh < 64; sh <<= 1) t += __shfl_xor(t, sh);
        if (lane == 0) dwr[wave * CH * CH + i] = t;
    }
    __syncthreads();
    for (int i = tid; i < CH * CH; i += NTB) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NWB; ++w) t += dwr[w * CH * CH + i];
        atomicAdd(bp.dw + (size_t)g * CH * CH + i, t);
    }
    for (int i = tid; i < CH * cq * ckp; i += NTB) {
        const int a = i / (cq * ckp), r = (i / ckp) % cq, c = i % ckp;
        if (c < ck) atomicAdd(bp.dtheta + ((size_t)(h0 + a) * cq + r) * ck + c, dth[i] * bp.inv_log2e);
    }
}

}  // namespace bwd

bwd::BwdFn find_launch_bwd(int dtype_bf16, int d, int ch, int cq, int ck, int exact);
// find_launch_bwd picks a main kernel with compile-time stencil sizes (whose
// convolved-map recompute runs on the matrix cores)
bool bwd_fixed_sizes(int dtype_bf16, int d, int ch, int cq, int ck);
hipError_t launch_fill_zero(const bwd::ZeroList &z, hipStream_t s);

}  // namespace mta
