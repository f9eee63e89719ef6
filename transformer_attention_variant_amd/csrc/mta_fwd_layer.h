// mta_fwd_layer.h — the general MTA layer on gfx950: every stage of "Putting
// Everything Together" (page "Multi-Token Attention — Paper Graph", section
// 3.4), each optional:
//
//   L = S,  or  Conv2d_theta1(Mask_0(S))  (Eq. 4's indicator instead of Mask_0
//       when `exact`),  or the 3D convolution  L^a = sum_b Conv2d_theta3[a][b](.)
//   L = head mix w_pre (L)                         (not with the 3D kernel)
//   P = softmax(Mask_-inf(L))
//   P = head mix w_post (P)                        (Eq. 7)
//   P = Mask_0(Conv2d_theta2(P))                    (key-query conv after the softmax)
//   P = head mix w_post2 (P)                       (the repeated head convolution)
//   O = P V;  GroupNorm over d x head factor.
//
// One workgroup (4 waves) owns (batch b, head group g, 64 query rows) and walks
// the causal key tiles twice (statistics, then probabilities).  Per key tile:
//   * the logits S of one source head over the rows and keys the stages reach
//     (the tile plus the post-softmax convolution's halo plus the pre-softmax
//     convolution's halo) are computed on the matrix cores into LDS;
//   * the pre-softmax convolution (fp32 VALU, 16 outputs per lane-task) writes
//     each head's map L over the tile plus the post-softmax halo into that
//     head's LDS buffer (the 3D kernel adds every source head's term into
//     every output head's buffer, one source head at a time);
//   * head mixes run elementwise across the group's buffers;
//   * pass 1 keeps each row's (max, sum) online; pass 2 turns L into
//     probabilities in place, convolves them (lane = one row, 16 keys: the
//     A-operand slots of the P.V MFMA), applies Mask_0 and the last head mix in
//     registers, and multiplies by V on the matrix cores.
#pragma once

#include "mta_launch.h"

namespace mta {
namespace layer {

constexpr int NT = 256;

struct LParams {
    const void *q, *k, *v;
    void *out;
    const float *kq_pre, *head_pre, *conv3d, *head_post, *kq_post, *head_post2;
    const float *gn_w, *gn_b, *gate;
    int H, T, G, units, n_qt;
    int cq1, ck1, cq2, ck2;    // pre-softmax (kq_pre / conv3d) and post-softmax kernel sizes
    int pre;                   // 0 none, 1 key-query kernel per head, 2 3D kernel
    int exact;
    // geometry (host-computed): L rows/cols (tile + post halo) and S rows/cols
    int h2, l2, h1, l1;        // rows above / keys left of the tile: post stage, pre stage
    int nLr, nLc, lpitch;      // L map: rows, columns, floats per row
    int nSrb, nScb, spitch;    // S tile: 16-row blocks, 16-column blocks, floats per row
    int ck1p, ck2p;            // kernel rows padded to 4
    float sc, eps, depth_scale;
};

struct LLayout {
    int s_off, l_off, st_off, th1_off, th2_off, w_off, v_off, total;
};

template <typename DT, int D>
__host__ __device__ inline LLayout llayout(const LParams &p, int CH)
{
    LLayout L;
    int o = 0;
    // the logit tile of the pre-softmax convolution and the V tile of P.V are
    // never live together: one region
    const int sbytes = p.nSrb * 16 * p.spitch * 4, vbytes = vbuf_bytes<DT, D>();
    L.s_off = o;
    L.v_off = o;   o += sbytes > vbytes ? sbytes : vbytes;
    L.l_off = o;   o += CH * p.nLr * p.lpitch * 4;
    L.st_off = o;  o += 2 * CH * ((p.nLr + 3) & ~3) * 4;
    const int n1 = p.pre == 2 ? CH * CH * p.cq1 * p.ck1p : CH * p.cq1 * p.ck1p;
    L.th1_off = o; o += ((n1 + 3) & ~3) * 4;
    L.th2_off = o; o += ((CH * p.cq2 * p.ck2p + 3) & ~3) * 4;
    L.w_off = o;   o += 3 * ((CH * CH + 3) & ~3) * 4;
    L.total = o;
    return L;
}

// Logits of one head into an LDS tile whose row 0 is query r0 and column 0 is
// key c0: x = S*log2(e)/sqrt(d) where 0 <= query < T, 0 <= key < T and (unless
// `raw`) key <= query (Mask_0); 0 elsewhere.  Wave w takes the row blocks
// w, w+4, ... (one Q fragment each) and every column block; rows >= nrows of
// the last block are not stored.
template <typename DT, int D>
__device__ inline void s_tile(float *buf, int pitch, int nrb, int ncb, int nrows, const DT *qh, const DT *kh,
                              int r0, int c0, int T, float sc, bool raw, int wave, int lane)
{
    typedef typename FragOf<DT, D>::type Frag;
    // one 16-row block: products with the column blocks [cb0, ncb) step cstep;
    // the K fragments of the next two blocks are requested before each
    // product (the loads come from L2 / HBM)
    auto row_block = [&](int rb, int cb0, int cstep) {
        Frag qf, kf, k1;
        const int qi = r0 + 16 * rb + (lane & 15);
        load_frag<D>(qf, qh, qi, T, lane);
        load_frag<D>(kf, kh, c0 + 16 * cb0 + (lane & 15), T, lane);
        if (cb0 + cstep < ncb) load_frag<D>(k1, kh, c0 + 16 * (cb0 + cstep) + (lane & 15), T, lane);
        for (int cb = cb0; cb < ncb; cb += cstep) {
            Frag k2;
            if (cb + 2 * cstep < ncb) load_frag<D>(k2, kh, c0 + 16 * (cb + 2 * cstep) + (lane & 15), T, lane);
            const f32x4 acc = qk_mfma<D>(kf, qf);
            kf = k1;
            k1 = k2;
            const int e0 = 16 * cb + 4 * (lane >> 4);
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kj = c0 + e0 + r;
                const bool ok = qi >= 0 && qi < T && kj >= 0 && kj < T && (raw || kj <= qi);
                o[r] = ok ? acc[r] * sc : 0.f;
            }
            if (16 * rb + (lane & 15) < nrows)
                *reinterpret_cast<f32x4 *>(buf + (16 * rb + (lane & 15)) * pitch + e0) = o;
        }
    };
    // whole rounds of row blocks: one per wave; the remaining row blocks'
    // column blocks are dealt to the waves in turn
    const int full = nrb & ~3;
    for (int rb = wave; rb < full; rb += 4) row_block(rb, 0, 1);
    for (int rb = full; rb < nrb; ++rb)
        if (wave < ncb) row_block(rb, wave, 4);
}

// CQ1/CK1, CQ2/CK2: compile-time sizes of the pre- and post-softmax key-query
// kernels (0 = the runtime-sized stencil).
template <typename DT, int D, int CH, int CQ1, int CK1, int CQ2, int CK2>
__global__ void __launch_bounds__(NT) mta_fwd_layer(LParams p)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;  // longest rows first
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;

    const LLayout lay = llayout<DT, D>(p, CH);
    float *sraw = reinterpret_cast<float *>(smem + lay.s_off);
    float *lbuf = reinterpret_cast<float *>(smem + lay.l_off);
    float *st_m = reinterpret_cast<float *>(smem + lay.st_off);
    const int nLr4 = (p.nLr + 3) & ~3;
    float *st_il = st_m + CH * nLr4;
    float *th1 = reinterpret_cast<float *>(smem + lay.th1_off);
    float *th2 = reinterpret_cast<float *>(smem + lay.th2_off);
    float *wpre = reinterpret_cast<float *>(smem + lay.w_off);
    const int wstride = (CH * CH + 3) & ~3;
    float *wpost = wpre + wstride;
    float *wpost2 = wpost + wstride;
    DT *vbuf = reinterpret_cast<DT *>(smem + lay.v_off);

    const size_t hstride = (size_t)T * D;
    const DT *Q = reinterpret_cast<const DT *>(p.q);
    const DT *K = reinterpret_cast<const DT *>(p.k);
    const DT *V = reinterpret_cast<const DT *>(p.v);
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;

    // the group's kernels, rows padded to 4 (zeros)
    if (p.pre == 1) {
        for (int i = tid; i < CH * p.cq1 * p.ck1p; i += NT) {
            const int a = i / (p.cq1 * p.ck1p), r = (i / p.ck1p) % p.cq1, c = i % p.ck1p;
            th1[i] = c < p.ck1 ? p.kq_pre[((size_t)(h0 + a) * p.cq1 + r) * p.ck1 + c] : 0.f;
        }
    } else if (p.pre == 2) {
        for (int i = tid; i < CH * CH * p.cq1 * p.ck1p; i += NT) {
            const int ab = i / (p.cq1 * p.ck1p), r = (i / p.ck1p) % p.cq1, c = i % p.ck1p;
            th1[i] = c < p.ck1 ? p.conv3d[(((size_t)g * CH * CH + ab) * p.cq1 + r) * p.ck1 + c] : 0.f;
        }
    }
    if (p.kq_post) {
        for (int i = tid; i < CH * p.cq2 * p.ck2p; i += NT) {
            const int a = i / (p.cq2 * p.ck2p), r = (i / p.ck2p) % p.cq2, c = i % p.ck2p;
            th2[i] = c < p.ck2 ? p.kq_post[((size_t)(h0 + a) * p.cq2 + r) * p.ck2 + c] : 0.f;
        }
    }
    for (int i = tid; i < CH * CH; i += NT) {
        wpre[i] = p.head_pre ? p.head_pre[(size_t)g * CH * CH + i] : 0.f;
        wpost[i] = p.head_post ? p.head_post[(size_t)g * CH * CH + i] : 0.f;
        wpost2[i] = p.head_post2 ? p.head_post2[(size_t)g * CH * CH + i] : 0.f;
    }

    const int lr0 = i0 - p.h2;            // query of L row 0
    const int lc0 = 0 - p.l2;             // key of L column 0, relative to the key tile start
    const int sr0 = lr0 - p.h1;           // query of S row 0
    const int nlcb = (p.nLc + 15) / 16;   // 16-column chunks of L
    const int ntask = p.nLr * nlcb;

    // L of every head of the group for key tile j0 into lbuf
    auto compute_L = [&](int j0) {
        for (int s = 0; s < CH; ++s) {
            __syncthreads();  // sraw / lbuf free
            s_tile<DT, D>(sraw, p.spitch, p.nSrb, p.nScb, 16 * p.nSrb, Q + base0 + s * hstride,
                          K + base0 + s * hstride, sr0, j0 + lc0 - p.l1, T, p.sc, p.exact != 0, wave, lane);
            __syncthreads();
            for (int t = tid; t < ntask; t += NT) {
                const int rho = t / nlcb, cb = t % nlcb;
                const int qi = lr0 + rho;
                // window column w <-> key j0 + lc0 - l1 + 16cb + w; Eq. 4's indicator keeps key <= qi
                const int tlim = p.exact ? qi - (j0 + lc0 - p.l1 + 16 * cb) : (1 << 30);
                if (p.pre == 1) {
                    float o[16];
                    stencil16<CQ1, CK1>(sraw, p.spitch, rho + p.h1, 16 * cb, th1 + s * p.cq1 * p.ck1p, p.cq1,
                                        p.ck1, p.ck1p, tlim, o);
                    float *dst = lbuf + (s * p.nLr + rho) * p.lpitch + 16 * cb;
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[e] = o[e];
                } else {
                    // 3D kernel: source head s adds its term to every output head a
#pragma unroll
                    for (int a = 0; a < CH; ++a) {
                        float o[16];
                        stencil16<CQ1, CK1>(sraw, p.spitch, rho + p.h1, 16 * cb,
                                            th1 + (a * CH + s) * p.cq1 * p.ck1p, p.cq1, p.ck1, p.ck1p, tlim, o);
                        float *dst = lbuf + (a * p.nLr + rho) * p.lpitch + 16 * cb;
#pragma unroll
                        for (int e = 0; e < 16; ++e) dst[e] = (s == 0 ? 0.f : dst[e]) + o[e];
                    }
                }
            }
        }
        __syncthreads();
        if (p.head_pre) {
            for (int idx = tid; idx < p.nLr * p.nLc; idx += NT) {
                const int rho = idx / p.nLc, c = idx % p.nLc;
                float x[CH];
#pragma unroll
                for (int a = 0; a < CH; ++a) x[a] = lbuf[(a * p.nLr + rho) * p.lpitch + c];
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    float y = 0.f;
#pragma unroll
                    for (int s = 0; s < CH; ++s) y = __builtin_fmaf(wpre[a * CH + s], x[s], y);
                    lbuf[(a * p.nLr + rho) * p.lpitch + c] = y;
                }
            }
            __syncthreads();
        }
    };
    // no pre-softmax convolution: the L map is the logit tile itself
    auto compute_S_as_L = [&](int j0) {
        __syncthreads();
        for (int a = 0; a < CH; ++a)
            s_tile<DT, D>(lbuf + a * p.nLr * p.lpitch, p.lpitch, (p.nLr + 15) / 16, (p.nLc + 15) / 16, p.nLr,
                          Q + base0 + a * hstride, K + base0 + a * hstride, lr0, j0 + lc0, T, p.sc, true, wave,
                          lane);
        __syncthreads();
        if (p.head_pre) {
            for (int idx = tid; idx < p.nLr * p.nLc; idx += NT) {
                const int rho = idx / p.nLc, c = idx % p.nLc;
                float x[CH];
#pragma unroll
                for (int a = 0; a < CH; ++a) x[a] = lbuf[(a * p.nLr + rho) * p.lpitch + c];
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    float y = 0.f;
#pragma unroll
                    for (int s = 0; s < CH; ++s) y = __builtin_fmaf(wpre[a * CH + s], x[s], y);
                    lbuf[(a * p.nLr + rho) * p.lpitch + c] = y;
                }
            }
            __syncthreads();
        }
    };
    auto make_L = [&](int j0) {
        if (p.pre == 0) compute_S_as_L(j0);
        else compute_L(j0);
    };

    // ---------------- pass 1: row statistics over rows [lr0, i0 + 64) ------
    // slot t = tid + NT*k: L row t/4, keys 16*(t%4).. of the key tile
    constexpr int NSLOT = 2;  // nLr <= 128
    float sm[NSLOT][CH], sl[NSLOT][CH];
#pragma unroll
    for (int k2 = 0; k2 < NSLOT; ++k2)
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            sm[k2][a] = NEG_INF;
            sl[k2][a] = 0.f;
        }
    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        make_L(j0);
#pragma unroll
        for (int k2 = 0; k2 < NSLOT; ++k2) {
            const int t = tid + NT * k2;
            const int rho = t >> 2, q4 = t & 3;
            if (rho >= p.nLr) continue;
            const int qi = lr0 + rho;
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                float x[16];
                const float *src = lbuf + (a * p.nLr + rho) * p.lpitch + p.l2 + 16 * q4;
#pragma unroll
                for (int o = 0; o < 16; ++o) x[o] = src[o];
                stats_update(x, j0 + 16 * q4, qi, sm[k2][a], sl[k2][a]);
            }
        }
    }
    // merge the four lanes of a row (consecutive tids) and publish per row
#pragma unroll
    for (int k2 = 0; k2 < NSLOT; ++k2) {
        const int t = tid + NT * k2;
        const int rho = t >> 2;
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            float m = sm[k2][a], l = sl[k2][a];
#pragma unroll
            for (int sh = 1; sh <= 2; sh <<= 1) {
                const float m2 = __shfl_xor(m, sh), l2v = __shfl_xor(l, sh);
                const float mx = fmaxf(m, m2);
                if (mx != NEG_INF) {
                    l = (m == NEG_INF ? 0.f : l * __builtin_amdgcn_exp2f(m - mx)) +
                        (m2 == NEG_INF ? 0.f : l2v * __builtin_amdgcn_exp2f(m2 - mx));
                    m = mx;
                }
            }
            if ((t & 3) == 0 && rho < p.nLr) {
                // rows above the sequence start have no causal entry: zero padding
                const bool live = lr0 + rho >= 0 && m != NEG_INF;
                st_m[a * nLr4 + rho] = live ? m : 0.f;
                st_il[a * nLr4 + rho] = live ? 1.0f / l : 0.f;
            }
        }
    }
    __syncthreads();

    // ---------------- pass 2: probabilities, post stages, P V --------------
    f32x4 acc[CH][D / 16];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) acc[a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int io = wave * 16 + (lane & 15);  // the lane's output row within the tile
    const int jb = 16 * (lane >> 4);         // its first key within the key tile
    const int qabs = i0 + io;

    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        make_L(j0);
        // probabilities in place (0 outside 0 <= key <= query), then w_post
        for (int idx = tid; idx < p.nLr * p.nLc; idx += NT) {
            const int rho = idx / p.nLc, c = idx % p.nLc;
            const int qi = lr0 + rho, kj = j0 + lc0 + c;
            const bool ok = kj >= 0 && kj <= qi && qi >= 0;
            float x[CH];
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                const float l = lbuf[(a * p.nLr + rho) * p.lpitch + c];
                x[a] = ok ? __builtin_amdgcn_exp2f(l - st_m[a * nLr4 + rho]) * st_il[a * nLr4 + rho] : 0.f;
            }
            if (p.head_post) {
                float y[CH];
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    y[a] = 0.f;
#pragma unroll
                    for (int s = 0; s < CH; ++s) y[a] = __builtin_fmaf(wpost[a * CH + s], x[s], y[a]);
                }
#pragma unroll
                for (int a = 0; a < CH; ++a) x[a] = y[a];
            }
#pragma unroll
            for (int a = 0; a < CH; ++a) lbuf[(a * p.nLr + rho) * p.lpitch + c] = x[a];
        }
        __syncthreads();
        float pr[CH][16];
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            if (p.kq_post) {
                stencil16<CQ2, CK2>(lbuf + a * p.nLr * p.lpitch, p.lpitch, p.h2 + io, jb,
                                    th2 + a * p.cq2 * p.ck2p, p.cq2, p.ck2, p.ck2p, 1 << 30, pr[a]);
#pragma unroll
                for (int o = 0; o < 16; ++o) pr[a][o] = (j0 + jb + o <= qabs) ? pr[a][o] : 0.f;  // Mask_0
            } else {
                const float *src = lbuf + (a * p.nLr + p.h2 + io) * p.lpitch + p.l2 + jb;
#pragma unroll
                for (int o = 0; o < 16; ++o) pr[a][o] = src[o];
            }
        }
        if (p.head_post2) head_mix16<CH>(pr, wpost2);
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            __syncthreads();
            load_v_tile<D>(vbuf, V + base0 + a * hstride, j0, T, tid);
            __syncthreads();
            pv_mfma<D>(acc[a], pr[a], vbuf, lane);
        }
    }

    // ---------------- epilogue: GroupNorm over d, head factor, store -------
    DT *O = reinterpret_cast<DT *>(p.out);
    const int n = lane & 15;
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        const int h = h0 + a;
        const float *gw = p.gn_w + (size_t)h * D;
        const float *gb = p.gn_b + (size_t)h * D;
        const float hf = p.gate ? p.depth_scale / (1.0f + __expf(-p.gate[h])) : p.depth_scale;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) s += acc[a][nb][r];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 8);
            const float mu = s * (1.0f / D);
            float v2 = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const float dlt = acc[a][nb][r] - mu;
                v2 = __builtin_fmaf(dlt, dlt, v2);
            }
            v2 += __shfl_xor(v2, 1);
            v2 += __shfl_xor(v2, 2);
            v2 += __shfl_xor(v2, 4);
            v2 += __shfl_xor(v2, 8);
            const float rstd = 1.0f / __builtin_sqrtf(v2 * (1.0f / D) + p.eps);
            const int row = i0 + wave * 16 + 4 * (lane >> 4) + r;
            if (row < T) {
                DT *dst = O + ((size_t)b * p.H + h) * hstride + (size_t)row * D;
#pragma unroll
                for (int nb = 0; nb < D / 16; ++nb) {
                    const int col = nb * 16 + n;
                    const float y = ((acc[a][nb][r] - mu) * rstd * gw[col] + gb[col]) * hf;
                    dst[col] = cvt_out<DT>(y);
                }
            }
        }
    }
}

template <typename DT, int D, int CH, int CQ1 = 0, int CK1 = 0, int CQ2 = 0, int CK2 = 0>
hipError_t launch(const LParams &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_layer<DT, D, CH, CQ1, CK1, CQ2, CK2>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p);
    return hipGetLastError();
}

}  // namespace layer
}  // namespace mta
