// mta_fwd_rep.h — the repeated MTA convolution of the overall flow (page
// "Multi-Token Attention — Paper Graph", section 3.4, "Putting Everything
// Together: The Full MTA Module": a key-query convolution before the softmax,
// the head mix, then a second key-query convolution and head mix after it) on
// head-split waves, bf16, d = 128, c_h = 2, two-pass masks for the first
// convolution.  A workgroup owns one head pair (the group) and 64 query rows.
//
// The stages after the softmax are linear in the probabilities, so with
// P^b = softmax(Mask_-inf(Conv_{theta1^b}(Mask_0(S^b)))) the mixed map is
//   P3^c = Mask_0( sum_b Conv_{Theta[c][b]}(P^b) ),
//   Theta[c][b] = sum_a w2[c][a] w1[a][b] theta2^a        (Eq. 4, Eq. 7)
// and O^c = P3^c V^c: one 3D stencil over both heads' probabilities, no head
// mix left for the epilogue.  The second convolution reads the probabilities
// of c_q2 - 1 rows above each row, normalised, so every row's softmax
// statistics must be known before any probability is formed: two passes over
// the key tiles.
//   Pass 1 — statistics: per key tile the logit tile of the 64 rows and the 16
//     rows above them (80 x 80: keys j0 - 8 ...), the first convolution over the
//     tile's 64 keys for all 80 rows, Mask_-inf, and a running maximum and sum
//     per row.
//   Pass 2 — per key tile: the logit tile (80 x 96: keys j0 - 16 ...), the first
//     convolution over 80 keys (j0 - 8 ...) for all 80 rows, probabilities with
//     pass 1's statistics (fp16 tile), the 3D second convolution over the 64
//     rows and keys, Mask_0, P.V.
// Both convolutions run on the matrix cores with fp16 operands (the logits or
// probabilities and the taps rounded to nearest, 11 significant bits) and fp32
// accumulation, one product per kernel row and 16-key output block, as in the
// head-split kernel.  The centre tap of the first convolution (the largest tap
// of a kernel near the identity) stays out of the fp16 band and is applied to
// the float32 logit, which the lane gets from its partner lane 32 away (same
// row, eight keys over) for its own rows and from a small float32 plane in LDS
// for the rows above the tile, so that its term keeps float32 accuracy at any
// logit size.
#pragma once

#include "mta_fwd_v4.h"

namespace mta {
namespace rep {

using tile::barrier_lds;
using tile::swz_k;
using tile::vread_tr4;
using v4::f16_range;
using v4::f16_t;
using v4::f16x4;
using v4::f16x8;
using v4::qk;
using v4::row_max4;
using v4::row_sum4;
using v4::u32x2;
using v4::wait_vm_all;

constexpr int NT = 512;  // 8 waves, two per SIMD
constexpr int CH = 2;
constexpr int D = 128;
constexpr int KR1 = 80;   // pass 1: K rows per head (keys j0 - 8 .. j0 + 71)
constexpr int KR2 = 96;   // pass 2: K rows per head (keys j0 - 16 .. j0 + 79)
constexpr int XP1 = 80;   // pass 1 logit tile pitch (fp16; 16-byte chunks per row = 2 mod 4)
constexpr int XP2 = 112;  // pass 2 logit tile pitch (96 columns used)
constexpr int PT = 80;    // probability tile pitch (80 columns: keys j0 - 8 .. j0 + 71)
constexpr int HCR = 8;    // rows above the tile whose first-convolution output is used (c_q2 - 1 <= 8)
constexpr int HCP = 96;   // float32 pitch of their centre-tap plane

struct RParams {
    const void *q, *k, *v;
    const float *theta1;  // [H][c_q1][c_k1]: before the softmax
    const float *w1;      // [H/2][2][2] head mix after the softmax, or null (identity)
    const float *theta2;  // [H][c_q2][c_k2]: after the softmax
    const float *w2;      // [H/2][2][2] the repeated head mix, or null (identity)
    const float *gn_w, *gn_b;
    const float *gate;    // [H] or null
    void *out;
    int H, T, G, units, n_qt;
    float sc;             // log2(e) / sqrt(d)
    float eps, depth_scale;
};

struct RLayout {
    int x_off, k_off, v_off, qh_off, pt_off, st_off, hp_off, th_off, hc_off, total;
};

template <int CQ1, int CK1, int CQ2, int CK2>
__host__ __device__ constexpr RLayout rlayout()
{
    RLayout L{};
    int o = 0;
    L.x_off = o;  o += CH * EXT_R * XP2 * 2;    // logit tiles (pass 1 uses pitch XP1)
    L.k_off = o;  o += CH * KR2 * D * 2;        // K tiles (swizzled rows)
    L.v_off = o;  o += CH * BN * D * 2;         // V tiles (swizzled rows)
    L.qh_off = o; o += CH * HALO * D * 2;       // Q rows above the query tile
    L.pt_off = o; o += CH * EXT_R * PT * 2;     // probability tiles (fp16)
    L.st_off = o; o += 2 * CH * EXT_R * 4;      // [h][row] maximum (log2 domain), 1 / sum
    L.hp_off = o; o += CH * 4 * 16 * 2 * 4;     // pass 1, rows above the tile: [h][key block][row][max, sum]
    L.th_off = o; o += (CH * CQ1 * ((CK1 + 3) & ~3) + CH * CH * CQ2 * ((CK2 + 3) & ~3)) * 4;
    L.hc_off = o; o += CH * HCR * HCP * 4;     // float32 logits of the lowest HCR rows above the tile
    L.total = o;
    return L;
}

// Output factor of head h: depth_scale, times sigmoid(gate[h]) with a gate.
__device__ inline float rhead_factor(const RParams &p, int h)
{
    if (!p.gate) return p.depth_scale;
    return p.depth_scale / (1.0f + __expf(-p.gate[h]));
}

// Banded kernel matrix rows of one kernel row (MFMA A operand, fp16): row m =
// lane%16 is output key 16t + m of a block, column k = 8*(lane/16) + s of the
// 32-column window starting 8 keys left of the block, so j' = m + 8 - k.
// nocentre: the centre tap (j' = 0) left out (applied in float32 by the caller).
template <int CK>
__device__ inline f16x8 band(const float *th_row, float kap, int lane, bool nocentre = false)
{
    const int l16 = lane & 15, g4 = lane >> 4;
    f16x8 r;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
        const int jj = l16 + 8 - (8 * g4 + s8) + CK / 2;
        const float t = (jj >= 0 && jj < CK && !(nocentre && jj == CK / 2)) ? th_row[jj] : 0.f;
        r[s8] = (f16_t)f16_range(t * kap);
    }
    return r;
}

// One 16-key output block of a stencil for the lane's row rho of an fp16 tile
// (pitch P): the window starts at tile column col0; rows above the tile are
// clamped to row 0 (they only feed rows whose results are not used).
template <int CQ, int P>
__device__ inline f32x4 sten(const f16_t *x, int rho, const f16x8 (&tf)[CQ], int col0, int g4, f32x4 acc)
{
#pragma unroll
    for (int ip = 0; ip < CQ; ++ip) {
        int r = rho - ip;
        r = r < 0 ? 0 : r;
        const f16x8 xv = *reinterpret_cast<const f16x8 *>(x + r * P + col0 + 8 * g4);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(tf[ip], xv, acc, 0, 0, 0);
    }
    return acc;
}

// A 16x16 logit block (lane: tile row 16rb + lane%16, keys k0 + 4*(lane/16) + r)
// with Mask_0 and the zero padding outside [0, T), as fp16, stored 8 bytes per
// lane; returns the masked logits in float32.
template <int P>
__device__ inline f32x4 store_logits(f16_t *x, int rb, int cb, f32x4 acc, int qi, int k0, int T, int lane)
{
    const int l16 = lane & 15, g4 = lane >> 4;
    f16x4 h;
    f32x4 xs;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int kj = k0 + 4 * g4 + r;
        const bool ok = kj >= 0 && kj <= qi && qi >= 0 && qi < T;
        xs[r] = ok ? acc[r] : 0.f;
        h[r] = (f16_t)f16_range(xs[r]);
    }
    *reinterpret_cast<u32x2 *>(x + (16 * rb + l16) * P + 16 * cb + 4 * g4) = __builtin_bit_cast(u32x2, h);
    return xs;
}

// The centre logits of a 16-key stencil output block whose window starts at
// logit column block u (output keys 8 + 16u + 4*(lane/16) + r of the row): for
// lanes 0..31 they sit in block u of the partner lane 32 above, for lanes
// 32..63 in block u + 1 of the partner lane 32 below (one permlane32 swap).
__device__ inline f32x4 centre_pair(f32x4 xu, f32x4 xu1, int lane)
{
    f32x4 c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(xu[r]), __float_as_uint(xu1[r]), false, false);
        c[r] = __uint_as_float(lane < 32 ? w[1] : w[0]);
    }
    return c;
}


// DMA of NROWS consecutive rows of a K or V tile for both heads (as
// v4::dma_pair).  The lane index passes through an empty asm, so that the
// per-piece lane offsets are computed where they are used: held across the
// loop they were spilled, and each reload waited for every DMA in flight.
template <bool VTILE, int NROWS>
__device__ inline void dma(bf16_t *lds, const bf16_t *g, size_t hstride, int key0, int T, int wave, int lane)
{
    v4::dma_pair<VTILE, NROWS>(lds, g, hstride, key0, T, wave, v4::fresh(lane));
}

// Running maximum and sum (log2 domain) over n values; a finite floor instead
// of -inf keeps l = 0 for a lane that has seen no causal key.
__device__ inline void online(float &m, float &l, const float *v, int n)
{
    float mx = m;
    for (int o = 0; o < n; ++o) mx = fmaxf(mx, v[o]);
    float s = 0.f;
    for (int o = 0; o < n; ++o) s += __builtin_amdgcn_exp2f(v[o] - mx);  // exp2(-inf) = 0
    l = __builtin_fmaf(l, __builtin_amdgcn_exp2f(m - mx), s);
    m = mx;
}

template <int CQ1, int CK1, int CQ2, int CK2>
__global__ void __launch_bounds__(NT, 1) mta_fwd_rep(RParams p)
{
    static_assert(CK1 <= 17 && CK2 <= 17, "32-column stencil windows");
    static_assert(CQ1 + CQ2 - 2 <= HALO, "the rows above the tile that both convolutions reach");
    static_assert(CQ2 - 1 <= HCR, "the centre-tap plane covers the rows above the tile that are used");
    constexpr int CK1P = (CK1 + 3) & ~3, CK2P = (CK2 + 3) & ~3;
    constexpr float FLOOR = -1e30f;
    constexpr RLayout lay = rlayout<CQ1, CK1, CQ2, CK2>();
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    f16_t *xbuf = reinterpret_cast<f16_t *>(smem + lay.x_off);
    bf16_t *kbuf = reinterpret_cast<bf16_t *>(smem + lay.k_off);
    bf16_t *vbuf = reinterpret_cast<bf16_t *>(smem + lay.v_off);
    bf16_t *qhbuf = reinterpret_cast<bf16_t *>(smem + lay.qh_off);
    f16_t *ptile = reinterpret_cast<f16_t *>(smem + lay.pt_off);
    float *stm = reinterpret_cast<float *>(smem + lay.st_off);  // [h][row]
    float *stil = stm + CH * EXT_R;                             // [h][row]
    float *hpart = reinterpret_cast<float *>(smem + lay.hp_off);
    float *th1 = reinterpret_cast<float *>(smem + lay.th_off);  // [h][row][col]
    float *th2 = th1 + CH * CQ1 * CK1P;                         // [c][b][row][col]
    float *hcen = reinterpret_cast<float *>(smem + lay.hc_off); // [h][row - (HALO - HCR)][col]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave & 3, hs = wave >> 2;  // row block; head (logits, stencils, P.V)
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM, T = p.T;
    const size_t hstride = (size_t)T * D;
    const int h0 = 2 * g;
    const size_t base = ((size_t)b * p.H + h0) * hstride;
    const bf16_t *Q = reinterpret_cast<const bf16_t *>(p.q) + base;
    const bf16_t *K = reinterpret_cast<const bf16_t *>(p.k) + base;
    const bf16_t *V = reinterpret_cast<const bf16_t *>(p.v) + base;

    // pass 1's first K tiles and the Q rows above the query tile (both heads);
    // this wave's own Q rows of head hs in registers; the kernels
    dma<false, KR1>(kbuf, K, hstride, -8, T, wave, lane);
    v4::dma_pair<false, HALO>(qhbuf, Q, hstride, i0 - HALO, T, wave, lane);
    const int qown_row = i0 + 16 * rw + l16;
    const bf16_t *qrow = Q + hs * hstride + (size_t)(qown_row < T ? qown_row : T - 1) * D + 32 * g4;
    QFrag<D> qown;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) qown.x[t] = *reinterpret_cast<const bf16x8 *>(qrow + 8 * t);
    for (int i = tid; i < CH * CQ1 * CK1P; i += NT) {
        const int a = i / (CQ1 * CK1P), r = (i / CK1P) % CQ1, c = i % CK1P;
        th1[i] = c < CK1 ? p.theta1[((size_t)(h0 + a) * CQ1 + r) * CK1 + c] : 0.f;
    }
    // Theta[c][b] = sum_a w2[c][a] w1[a][b] theta2^a (an absent mix is the identity)
    for (int i = tid; i < CH * CH * CQ2 * CK2P; i += NT) {
        const int cb = i / (CQ2 * CK2P), r = (i / CK2P) % CQ2, col = i % CK2P;
        const int c = cb / CH, bb = cb % CH;
        float v = 0.f;
        if (col < CK2) {
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                const float w2 = p.w2 ? p.w2[((size_t)g * CH + c) * CH + a] : (c == a ? 1.f : 0.f);
                const float w1 = p.w1 ? p.w1[((size_t)g * CH + a) * CH + bb] : (a == bb ? 1.f : 0.f);
                v = __builtin_fmaf(w2 * w1, p.theta2[((size_t)(h0 + a) * CQ2 + r) * CK2 + col], v);
            }
        }
        th2[i] = v;
    }
    wait_vm_all();
    __syncthreads();

    // banded matrices of the first kernel of head hs (log2(e)/sqrt(d) folded
    // in: the logit tiles hold raw Q K^T; the centre tap left out)
    f16x8 tf1[CQ1];
#pragma unroll
    for (int ip = 0; ip < CQ1; ++ip) tf1[ip] = band<CK1>(th1 + (hs * CQ1 + ip) * CK1P, p.sc, lane, ip == 0);
    // the first kernel's centre tap (left out of its banded matrices), applied
    // to the float32 logits
    const float c00 = th1[hs * CQ1 * CK1P + CK1 / 2] * p.sc;

    int koff[4];  // swizzled chunk offsets of the K / Q-halo fragment reads
#pragma unroll
    for (int t = 0; t < 4; ++t) koff[t] = 8 * ((4 * g4 + t) ^ swz_k(l16));
    auto kload = [&](QFrag<D> &f, const bf16_t *rows, int cb) {
#pragma unroll
        for (int t = 0; t < 4; ++t) f.x[t] = *reinterpret_cast<const bf16x8 *>(rows + 16 * cb * D + koff[t]);
    };
    // Q rows above the tile, head hs (the halo blocks of each wave are of its
    // own head), read from LDS where used
    const bf16_t *qhrows = qhbuf + (hs * HALO + l16) * D;
    const int qh = i0 - HALO + l16;  // the lane's row above the tile
    const int rho = HALO + 16 * rw + l16;  // the lane's own tile row
    f16_t *xo = xbuf + hs * EXT_R * XP2;  // head hs's logit tile (pass 1: pitch XP1)
    // the lane's row of the centre-tap plane (rows above the tile; the lanes of
    // the rows that are not used read row 0 and write nothing)
    float *hcrow = hcen + (hs * HCR + (l16 >= HALO - HCR ? l16 - (HALO - HCR) : 0)) * HCP;
    const bool hcw = l16 >= HALO - HCR;

    // ---------------- pass 1: softmax statistics of every tile row ----------------
    float m1 = FLOOR, l1 = 0.f, m2 = FLOOR, l2 = 0.f;  // own row; row above the tile (key block rw)
    for (int t = 0; t <= qt; ++t) {
        const int j0 = t * BN;
        if (t > 0) {
            wait_vm_all();
            __syncthreads();  // K(t) in LDS; the stencil reads of t - 1 are done
        }
        f32x4 cen[4];  // centre-tap terms of the own rows' four output blocks (float32)
        {
            const bf16_t *kh = kbuf + hs * KR1 * D + l16 * D;
            QFrag<D> kf;
            f32x4 xp;
#pragma unroll
            for (int cb = 0; cb < 5; ++cb) {
                kload(kf, kh, cb);
                const f32x4 x = store_logits<XP1>(xo, 1 + rw, cb, qk(kf, qown), qown_row, j0 - 8 + 16 * cb, T, lane);
                if (cb > 0) cen[cb - 1] = c00 * centre_pair(xp, x, lane);
                xp = x;
            }
            for (int cb = rw; cb < 5; cb += 4) {
                QFrag<D> hq;
                kload(hq, qhrows, 0);
                kload(kf, kh, cb);
                const f32x4 x = store_logits<XP1>(xo, 0, cb, qk(kf, hq), qh, j0 - 8 + 16 * cb, T, lane);
                if (hcw) *reinterpret_cast<f32x4 *>(hcrow + 16 * cb + 4 * g4) = x;
            }
        }
        barrier_lds();  // logit tiles and the centre-tap plane published; the K buffer is free
        if (t < qt) dma<false, KR1>(kbuf, K, hstride, j0 + BN - 8, T, wave, lane);
        // own rows: the 64 keys of the tile
        float c[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 a = sten<CQ1, XP1>(xo, rho, tf1, 16 * u, g4, cen[u]);
#pragma unroll
            for (int r = 0; r < 4; ++r) c[4 * u + r] = (j0 + 16 * u + 4 * g4 + r <= qown_row) ? a[r] : NEG_INF;
        }
        online(m1, l1, c, 16);
        // the row above the tile: key block rw
        {
            const f32x4 hc = *reinterpret_cast<const f32x4 *>(hcrow + 16 * rw + 8 + 4 * g4);
            f32x4 h0;
#pragma unroll
            for (int r = 0; r < 4; ++r) h0[r] = c00 * hc[r];
            const f32x4 a = sten<CQ1, XP1>(xo, l16, tf1, 16 * rw, g4, h0);
            float w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = (j0 + 16 * rw + 4 * g4 + r <= qh) ? a[r] : NEG_INF;
            online(m2, l2, w, 4);
        }
    }
    {
        // merge the four lanes of each row, then the four key blocks of the rows above the tile
        const float mo = row_max4(m1), lo = row_sum4(l1 * __builtin_amdgcn_exp2f(m1 - mo));
        const float mh = row_max4(m2), lh = row_sum4(l2 * __builtin_amdgcn_exp2f(m2 - mh));
        if (g4 == 0) {
            stm[hs * EXT_R + rho] = mo;
            stil[hs * EXT_R + rho] = lo > 0.f ? 1.0f / lo : 0.f;
            hpart[((hs * 4 + rw) * 16 + l16) * 2 + 0] = mh;
            hpart[((hs * 4 + rw) * 16 + l16) * 2 + 1] = lh;
        }
    }
    __syncthreads();  // pass 1 is done with the logit and K buffers; partial statistics published
    dma<false, KR2>(kbuf, K, hstride, -16, T, wave, lane);  // pass 2's first K tiles
    if (tid < CH * 16) {
        const int h = tid >> 4, r = tid & 15;
        float mr = FLOOR;
#pragma unroll
        for (int k = 0; k < 4; ++k) mr = fmaxf(mr, hpart[((h * 4 + k) * 16 + r) * 2]);
        float lr = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            lr = __builtin_fmaf(hpart[((h * 4 + k) * 16 + r) * 2 + 1],
                                __builtin_amdgcn_exp2f(hpart[((h * 4 + k) * 16 + r) * 2] - mr), lr);
        stm[h * EXT_R + r] = mr;
        stil[h * EXT_R + r] = lr > 0.f ? 1.0f / lr : 0.f;
    }
    wait_vm_all();
    __syncthreads();
    // statistics of the lane's own row and of its row above the tile (head hs)
    const float sm_o = stm[hs * EXT_R + rho], sil_o = stil[hs * EXT_R + rho];
    const float sm_h = stm[hs * EXT_R + l16], sil_h = stil[hs * EXT_R + l16];

    // ---------------- pass 2: probabilities, second convolution, P.V ----------------
    // wave (rw, s) forms output head s's mixed map for its 16 rows and multiplies
    // it by V^s over all 128 d-columns: the stencil's output layout is the P.V
    // A operand, so the map never leaves the registers
    f32x4 U[8];  // rows 16rw + 4g4 + r, d-columns 16nb + l16 of output head hs
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) U[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // banded matrices of the 3D kernel into output head hs
    f16x8 tf2[CH][CQ2];
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
        for (int ip = 0; ip < CQ2; ++ip) tf2[s][ip] = band<CK2>(th2 + ((hs * CH + s) * CQ2 + ip) * CK2P, 1.f, lane);

    for (int t = 0; t <= qt; ++t) {
        const int j0 = t * BN;
        f32x4 cen[5];  // centre-tap terms of the own rows' five output blocks (float32)
        if (t > 0) {
            wait_vm_all();  // K(t): this wave's pieces
            barrier_lds();  // A: K(t) in LDS; P.V of t - 1 (its V reads) and the second convolution are done
        }
        dma<true, BN>(vbuf, V, hstride, j0, T, wave, lane);  // V(t): four pieces per wave
        f16_t *po = ptile + hs * EXT_R * PT;
        const bf16_t *vh = vbuf + hs * BN * D;
        // probabilities of one output block of the first convolution (tile row
        // rr, query qi, keys k0 + 4*(lane/16) + r): exp2(C - m) / l with Mask_-inf
        // and the zero padding of the second convolution; entries whose exp2 may
        // be out of range are selected away, never multiplied
        auto to_prob = [&](f32x4 a, int rr, int qi, int k0, int col0, float m, float il) {
            f16x4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kj = k0 + 4 * g4 + r;
                const bool ok = kj >= 0 && kj <= qi && qi >= 0 && qi < T;
                const float e = __builtin_amdgcn_exp2f(a[r] - m) * il;
                h[r] = (f16_t)(ok ? e : 0.f);
            }
            *reinterpret_cast<u32x2 *>(po + rr * PT + col0 + 4 * g4) = __builtin_bit_cast(u32x2, h);
        };
        {
            // logits: own row block (six column blocks) and the row block above
            // the tile (column blocks rw, rw + 4 of head hs); keys j0 - 16 ...;
            // the float32 centre logits of the own rows' five output blocks kept
            // in registers, those of the rows above in the centre-tap plane
            const bf16_t *kh = kbuf + hs * KR2 * D + l16 * D;
            QFrag<D> kf;
            f32x4 xp;
#pragma unroll
            for (int cb = 0; cb < 6; ++cb) {
                kload(kf, kh, cb);
                const f32x4 x = store_logits<XP2>(xo, 1 + rw, cb, qk(kf, qown), qown_row, j0 - 16 + 16 * cb, T, lane);
                if (cb > 0) cen[cb - 1] = c00 * centre_pair(xp, x, lane);
                xp = x;
            }
            for (int cb = rw; cb < 6; cb += 4) {
                QFrag<D> hq;
                kload(hq, qhrows, 0);
                kload(kf, kh, cb);
                const f32x4 x = store_logits<XP2>(xo, 0, cb, qk(kf, hq), qh, j0 - 16 + 16 * cb, T, lane);
                if (hcw) *reinterpret_cast<f32x4 *>(hcrow + 16 * cb + 4 * g4) = x;
            }
        }
        barrier_lds();  // B: logit tiles and the centre-tap plane published; the K buffer is free
        if (t < qt) dma<false, KR2>(kbuf, K, hstride, j0 + BN - 16, T, wave, lane);  // K(t+1): six pieces per wave
        // first convolution over keys j0 - 8 ... j0 + 71 (five output blocks)
        // -> probabilities: own rows, and output blocks rw, rw + 4 of the rows above
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const f32x4 a = sten<CQ1, XP2>(xo, rho, tf1, 16 * u, g4, cen[u]);
            to_prob(a, rho, qown_row, j0 - 8 + 16 * u, 16 * u, sm_o, sil_o);
        }
        for (int u = rw; u < 5; u += 4) {
            const f32x4 hc = *reinterpret_cast<const f32x4 *>(hcrow + 16 * u + 8 + 4 * g4);
            f32x4 h0;
#pragma unroll
            for (int r = 0; r < 4; ++r) h0[r] = c00 * hc[r];
            const f32x4 a = sten<CQ1, XP2>(xo, l16, tf1, 16 * u, g4, h0);
            to_prob(a, l16, qh, j0 - 8 + 16 * u, 16 * u, sm_h, sil_h);
        }
        // V(t) has landed (issued before K(t+1), whose six pieces may stay in flight)
        if (t < qt)
            __builtin_amdgcn_s_waitcnt(0x0f76);  // vmcnt(6)
        else
            wait_vm_all();
        barrier_lds();  // C: probability tiles and V(t) published; the logit tiles are free
        // second convolution (3D: both source heads into output head hs), own
        // rows, the tile's 64 keys; Mask_0 on the diagonal tile; then P.V
        f32x4 acc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CH; ++s)
                acc[u] = sten<CQ2, PT>(ptile + s * EXT_R * PT, rho, tf2[s], 16 * u, g4, acc[u]);
        }
        bf16x8 av[2];  // keys 4g4 + r and 16 + 4g4 + r (slots 0-3, 4-7) of key halves 0 and 1
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                av[u >> 1][4 * (u & 1) + r] = (bf16_t)((j0 + 16 * u + 4 * g4 + r <= qown_row) ? acc[u][r] : 0.f);
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) {
            const int kb0 = 32 * cs + 4 * g4;  // keys of slots 0-3 and 4-7, in the producing lanes' order
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const tile::s16x4 u0 = vread_tr4(vh, kb0, 16 * nb, l16);
                const tile::s16x4 u1 = vread_tr4(vh, kb0 + 16, 16 * nb, l16);
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 uu = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                U[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[cs], __builtin_bit_cast(bf16x8, uu), U[nb], 0, 0,
                                                                0);
            }
        }
    }

    // ---------------- epilogue: GroupNorm over d (inside the wave), head factor, store -------
    float mu[4], rstd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) sum += U[nb][r];
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        sum += __shfl_xor(sum, 4);
        sum += __shfl_xor(sum, 8);
        mu[r] = sum * (1.0f / D);
        float v2s = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const float dl = U[nb][r] - mu[r];
            v2s = __builtin_fmaf(dl, dl, v2s);
        }
        v2s += __shfl_xor(v2s, 1);
        v2s += __shfl_xor(v2s, 2);
        v2s += __shfl_xor(v2s, 4);
        v2s += __shfl_xor(v2s, 8);
        rstd[r] = 1.0f / __builtin_sqrtf(v2s * (1.0f / D) + p.eps);
    }
    bf16_t *O = reinterpret_cast<bf16_t *>(p.out);
    const int h = h0 + hs;
    const float *gw = p.gn_w + (size_t)h * D;
    const float *gb = p.gn_b + (size_t)h * D;
    const float hf = rhead_factor(p, h);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = i0 + 16 * rw + 4 * g4 + r;
        if (row < T) {
            bf16_t *dst = O + ((size_t)b * p.H + h) * hstride + (size_t)row * D;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = 16 * nb + l16;
                dst[col] = (bf16_t)(((U[nb][r] - mu[r]) * rstd[r] * gw[col] + gb[col]) * hf);
            }
        }
    }
}

typedef hipError_t (*RepFn)(const RParams &p, int grid, size_t lds, hipStream_t s);

template <int CQ1, int CK1, int CQ2, int CK2>
hipError_t launch(const RParams &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_rep<CQ1, CK1, CQ2, CK2>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p);
    return hipGetLastError();
}

// LDS bytes of an instantiated size, 0 otherwise.
size_t lds_bytes(int cq1, int ck1, int cq2, int ck2);
// The instantiated kernel for (d, c_h, kernel sizes), or null.
RepFn find_launch(int d, int ch, int cq1, int ck1, int cq2, int ck2);

}  // namespace rep
}  // namespace mta
