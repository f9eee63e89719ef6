// mta_fwd_v3.h — one-pass MTA forward for the default placement: key-query
// convolution before the softmax (two-pass masks or Eq. 4's exact indicator),
// head mixing after it (page "Multi-Token Attention — Paper Graph", section
// 3.4, "Key-Query Convolution", "Head Mixing Convolution" Eq. 7, "Group
// Normalization with Sigmoid Gating").
//
// The two-pass kernels walk the key tiles twice: once for each row's softmax
// statistics, once for the probabilities.  Here the statistics are kept online
// instead.  Post-softmax mixing combines NORMALISED maps of different heads,
//   O^a = sum_b w_ab P^b V^a,  P^b = exp(C^b - m_b) / l_b,
// and l_b is only known at the end, so the kernel keeps one accumulator per
// (source head b, output head a):
//   U_{b,a} = sum_j exp(C^b_j - m_b) V^a_j   (rescaled when m_b grows),
//   O^a     = sum_b w_ab U_{b,a} / l_b        (in the epilogue).
// That costs c_h^2 accumulators and c_h times the P.V work, and saves the
// whole first pass (its logit tiles and convolutions).  c_h <= 2.
//
// Work split as in mta_fwd_v2.h: 8 waves, wave (rw, kh) owns query rows
// 16rw.. and, in the stencil, keys 32kh.. of each tile; in P.V the d-columns
// [kh*d/2, (kh+1)*d/2).  One phase per (key tile kt, head b), three barriers:
//   B1 | logit tile (kt, b) into LDS; P.V of tile kt-1 with V^b for every
//        source head (after rescaling the accumulators, in the phase of b = 0)
//   B2 | stencil of head b; partial row maximum of the wave's 32 keys -> LDS
//   B3 | row maximum of the tile, new running maximum m_b, rescale factor,
//        probabilities exp2(C - m_b) -> exchange buffer (tile parity)
#pragma once

#include "mta_fwd_v2.h"

namespace mta {
namespace v3 {

using v2::NT;
using v2::ColMask;
using v2::col_mask;
using v2::pitch_hl;

struct Layout {
    int s_off, k_off, qh_off, v_off, p_off, pm_off, al_off, th_off, w_off, gn_off, tf_off, total;
};

__host__ __device__ inline Layout layout(int D, int CH, int cq, int ck, int ncb)
{
    Layout L;
    int o = 0;
    L.s_off = o;  o += EXT_R * pitch_hl(ncb) * 2;           // logit tile (fp16)
    L.k_off = o;  o += ncb * 16 * D * 2;                    // K tile with key halo (bf16, swizzled rows)
    L.qh_off = o; o += CH * HALO * D * 2;                   // Q rows above the query tile, every head
    L.v_off = o;  o += BN * D * 2;                          // V tile (bf16, swizzled rows)
    L.p_off = o;  o += 2 * CH * 4 * 2 * 64 * 16;            // probabilities [parity][b][rw][chunk][lane] x 8 bf16
    L.pm_off = o; o += 2 * BM * 4;                          // partial row maxima [kh][row]
    L.al_off = o; o += CH * BM * 4;                         // rescale factors [b][row]; final 1/l
    L.th_off = o; o += ((CH * cq * ((ck + 3) & ~3) + 3) & ~3) * 4;
    L.w_off = o;  o += ((CH * CH + 3) & ~3) * 4;
    L.gn_off = o; o += 2 * CH * BM * 4;                     // GroupNorm partial sums; partial l
    L.tf_off = o; o += CH * cq * 64 * 16;                   // banded kernel matrices (MFMA A operands, fp16)
    L.total = o;
    return L;
}

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
typedef __attribute__((address_space(3))) void *lds_void_p;
typedef __attribute__((address_space(3))) v2::s16x4 *lds_s16x4_p;

__device__ inline int swz_k(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ inline int swz_v(int r) { return 2 * (r & 7); }

// Rows [0, nrows) of a tile: global rows key0 + row of the head slice g
// (clamped into [0, T); the rows outside are masked where they are used).
// nrows is a multiple of 4; the waves take the 1 KB pieces in turn.
template <bool VTILE>
__device__ inline void dma_tile(bf16_t *lds, const bf16_t *g, int key0, int nrows, int T, int wave, int lane)
{
    for (int i = wave; i < nrows / 4; i += NT / 64) {
        const int row = 4 * i + (lane >> 4), pc = lane & 15;
        const int c = pc ^ (VTILE ? swz_v(row) : swz_k(row));
        int key = key0 + row;
        key = key < 0 ? 0 : (key >= T ? T - 1 : key);
        __builtin_amdgcn_global_load_lds((const void *)(g + (size_t)key * 128 + 8 * c), (lds_void_p)(lds + 512 * i),
                                         16, 0, 0);
    }
}

// wait for this wave's outstanding global loads (the DMA tiles among them)
__device__ inline void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Workgroup barrier that publishes LDS writes but lets this wave's DMA tile
// loads stay in flight (a __syncthreads() fence would wait for them too).
// Only valid where no wave reads the DMA targets before the next full barrier,
// which waits for them.
__device__ inline void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Logit tile of one head: own-row block 1+rw from the Q fragment in registers,
// the halo block from the Q rows above the tile in LDS; K fragments from the
// swizzled K tile.  Work split and stores as in v2::logit_tile_lds.
template <int NCB, bool EX>
__device__ inline void logit_tile(v2::f16_t *x16, int ph, const QFrag<128> &qown, const bf16_t *qhalo,
                                  const bf16_t *kbuf, const Params &p, int i0, int j0, int rw, int kh, int lane)
{
    const int l16 = lane & 15, g4 = lane >> 4;
    const int fk = swz_k(l16);
    int off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) off[t] = 8 * ((4 * g4 + t) ^ fk);
    QFrag<128> kf;
#pragma unroll
    for (int cb = kh; cb < NCB; cb += 2) {
        const bf16_t *kr = kbuf + (16 * cb + l16) * 128;
#pragma unroll
        for (int t = 0; t < 4; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + off[t]);
        const f32x4 acc = qk_mfma<128>(kf, qown);
        v2::store_block_x<RAW>(x16, ph, 1 + rw, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane);
    }
    if (kh == 1 && p.c_q > 1) {
        QFrag<128> qh;
        const bf16_t *qr = qhalo + l16 * 128;
#pragma unroll
        for (int t = 0; t < 4; ++t) qh.x[t] = *reinterpret_cast<const bf16x8 *>(qr + off[t]);
#pragma unroll
        for (int cb = rw; cb < NCB; cb += 4) {
            const bf16_t *kr = kbuf + (16 * cb + l16) * 128;
#pragma unroll
            for (int t = 0; t < 4; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + off[t]);
            const f32x4 acc = qk_mfma<128>(kf, qh);
            v2::store_block_x<RAW>(x16, ph, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane);
        }
    }
}

// Transposing read of 4 keys kb + lane/4 (within the 16-lane group) of the
// swizzled V tile: element e of lane i is V[kb + e][d0 + i] (see v2::lds_read_tr4).
__device__ inline v2::s16x4 vread_tr4(const bf16_t *vbuf, int kb, int d0, int j)
{
    const int row = kb + (j >> 2), col = d0 + 4 * (j & 3);
    const bf16_t *a = vbuf + row * 128 + 8 * ((col >> 3) ^ swz_v(row)) + (col & 7);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)(a));
}

template <int D, int CH, int CQ, int CK, bool EXACT>
__global__ void __launch_bounds__(NT, 1) mta_fwd_v3(Params p)
{
    static_assert(CH == 1 || CH == 2, "one accumulator per (source, output) head pair: c_h <= 2");
    static_assert(CK <= 17, "matrix-core stencil: 32-column window");
    static_assert(D == 128, "tile swizzles assume 256-byte rows");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers and branches
    const int rw = wave & 3, kh = wave >> 2;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;
    constexpr int CKP = ((CK + 3) / 4) * 4;
    constexpr int NCB0 = (BN + CK - 1 + 15) / 16;
    constexpr int NCB = NCB0 < 5 ? 5 : NCB0;  // the stencil window spans >= 80 tile columns
    const int ph = pitch_hl(NCB);

    const Layout lay = layout(D, CH, CQ, CK, NCB);
    float *sbuf = reinterpret_cast<float *>(smem + lay.s_off);
    v2::f16_t *x16 = reinterpret_cast<v2::f16_t *>(sbuf);
    bf16_t *kbuf = reinterpret_cast<bf16_t *>(smem + lay.k_off);
    bf16_t *qhbuf = reinterpret_cast<bf16_t *>(smem + lay.qh_off);
    bf16_t *vbuf = reinterpret_cast<bf16_t *>(smem + lay.v_off);
    bf16x8 *pbuf = reinterpret_cast<bf16x8 *>(smem + lay.p_off);
    float *pm = reinterpret_cast<float *>(smem + lay.pm_off);   // [kh][row]
    float *al = reinterpret_cast<float *>(smem + lay.al_off);   // [b][row]
    float *th_s = reinterpret_cast<float *>(smem + lay.th_off);
    float *w_s = reinterpret_cast<float *>(smem + lay.w_off);
    float *gnx = reinterpret_cast<float *>(smem + lay.gn_off);  // [kh][a][row]
    v2::f16x8 *tf = reinterpret_cast<v2::f16x8 *>(smem + lay.tf_off);

    const size_t hstride = (size_t)T * D;
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;
    const bf16_t *Q = reinterpret_cast<const bf16_t *>(p.q) + base0;
    const bf16_t *K = reinterpret_cast<const bf16_t *>(p.k) + base0;
    const bf16_t *V = reinterpret_cast<const bf16_t *>(p.v) + base0;
    constexpr int krows = 16 * NCB;

    for (int i = tid; i < CH * CQ * CKP; i += NT) {
        const int a = i / (CQ * CKP), r = (i / CKP) % CQ, c = i % CKP;
        th_s[i] = c < CK ? p.theta[((size_t)(h0 + a) * CQ + r) * CK + c] : 0.f;
    }
    for (int i = tid; i < CH * CH; i += NT) w_s[i] = p.wmix[(size_t)g * CH * CH + i];
    __syncthreads();
    v2::build_theta_frags<CQ, CK>(tf, th_s, CH, tid, NT);

    const int io = 16 * rw + l16;  // the lane's stencil row within the query tile
    const int qabs = i0 + io;
    const int rho = HALO + io;
    const int col0 = 32 * kh + 8 * g4;
    // key (within the key tile) of each of the lane's 8 stencil outputs
    int ko[8];
#pragma unroll
    for (int o = 0; o < 8; ++o) ko[o] = 32 * kh + 16 * (o >> 2) + 4 * g4 + (o & 3);

    // K of key tile 0 (head 0) and the Q rows above the tile (every head) into
    // LDS; the wave's own Q rows of every head stay in registers throughout
    dma_tile<false>(kbuf, K, -p.hl, krows, T, wave, lane);
#pragma unroll
    for (int s = 0; s < CH; ++s) dma_tile<false>(qhbuf + s * HALO * D, Q + s * hstride, i0 - HALO, HALO, T, wave, lane);
    QFrag<D> qown[CH];
    {
        int qi = i0 + 16 * rw + l16;
        qi = qi < T ? qi : T - 1;  // rows past the end: masked in the logit tile
#pragma unroll
        for (int s = 0; s < CH; ++s)
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
                qown[s].x[t] = *reinterpret_cast<const bf16x8 *>(Q + s * hstride + (size_t)qi * D + 32 * g4 + 8 * t);
    }
    wait_vm();

    // U[b][a][nb][r]: rows 16rw + 4g4 + r, d-columns dbase + 16nb + l16
    f32x4 U[CH][CH][D / 32];
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) U[s][a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[CH], l_run[CH];  // running row maximum (log2 domain) and this lane's partial sum
#pragma unroll
    for (int s = 0; s < CH; ++s) {
        m_run[s] = NEG_INF;
        l_run[s] = 0.f;
    }
    const int dbase = kh * (D / 2);

    // P.V of one key tile with V^a in the V buffer, for every source head:
    // U[s][a] += P^s V^a.  The V fragments are read once and shared.
    auto pv = [&](int a, int par) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 av[CH];
#pragma unroll
            for (int s = 0; s < CH; ++s) av[s] = pbuf[(((par * CH + s) * 4 + rw) * 2 + c) * 64 + lane];
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
                // keys of slots 0-3 and 4-7, in the producing lanes' order
                const int kb0 = 32 * c + 4 * g4;
                const v2::s16x4 u0 = vread_tr4(vbuf, kb0, dbase + 16 * nb, l16);
                const v2::s16x4 u1 = vread_tr4(vbuf, kb0 + 16, dbase + 16 * nb, l16);
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 u = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                const bf16x8 bv = __builtin_bit_cast(bf16x8, u);
#pragma unroll
                for (int s = 0; s < CH; ++s)
                    U[s][a][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s], bv, U[s][a][nb], 0, 0, 0);
            }
        }
    };
    // bring every accumulator into the frame of the newest running maxima
    auto rescale = [&]() {
#pragma unroll
        for (int s = 0; s < CH; ++s) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = al[s * BM + 16 * rw + 4 * g4 + r];
#pragma unroll
            for (int a = 0; a < CH; ++a)
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) U[s][a][nb][r] *= f[r];
        }
    };

    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
#pragma unroll
        for (int s = 0; s < CH; ++s) {
            __syncthreads();  // B1: K^s(kt) and V^s(kt-1) are in LDS
            const int sn = (s + 1 < CH) ? s + 1 : 0;
            const int ktn = (s + 1 < CH) ? kt : kt + 1;
            logit_tile<NCB, EXACT>(x16, ph, qown[s], qhbuf + s * HALO * D,
                                   kbuf, p, i0, j0, rw, kh, lane);
            if (kt > 0) {
                if (s == 0) rescale();
                pv(s, (kt - 1) & 1);
            }
            __syncthreads();  // B2
            // the next phase (kt, s+1) or (kt+1, 0): its K tile and the V tile
            // its P.V reads go straight into LDS while this phase convolves
            if (ktn <= qt) dma_tile<false>(kbuf, K + sn * hstride, ktn * BN - p.hl, krows, T, wave, lane);
            if (ktn >= 1) dma_tile<true>(vbuf, V + sn * hstride, (ktn - 1) * BN, BN, T, wave, lane);

            float c[8];
            const int tl = EXACT ? qabs - (j0 - p.hl + col0) : (1 << 30);
            if (EXACT && j0 - p.hl + 32 * kh + 47 > i0 + 16 * rw)
                v2::stencil_mfma<CQ, true>(x16, ph, rho, kh, tf + s * CQ * 64, col_mask(tl), lane, c);
            else
                v2::stencil_mfma<CQ, false>(x16, ph, rho, kh, tf + s * CQ * 64, ColMask{}, lane, c);
            // Mask_-inf, then the maximum over this wave's 32 keys of the row
            float mx = NEG_INF;
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                c[o] = (j0 + ko[o] <= qabs) ? c[o] : NEG_INF;
                mx = fmaxf(mx, c[o]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g4 == 0) pm[kh * BM + io] = mx;
            barrier_lds();  // B3 (the DMA tiles stay in flight)
            // every row has a causal key in tile 0, so m_new is finite
            const float m_new = fmaxf(m_run[s], fmaxf(mx, pm[(kh ^ 1) * BM + io]));
            const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
            m_run[s] = m_new;
            float ls = 0.f;
            bf16x8 v8;
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const float e = __builtin_amdgcn_exp2f(c[o] - m_new);  // exp2(-inf) = 0 in the future
                ls += e;
                v8[o] = (bf16_t)e;
            }
            l_run[s] = __builtin_fmaf(l_run[s], alpha, ls);
            if (kh == 0 && g4 == 0) al[s * BM + io] = alpha;
            pbuf[((((kt & 1) * CH + s) * 4 + rw) * 2 + kh) * 64 + lane] = v8;
            wait_vm();
        }
    }
    // P.V of the last key tile, one output head at a time through the V buffer
    // (V^0 of the last tile arrived with the last phase)
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        __syncthreads();
        if (a == 0) rescale();
        pv(a, qt & 1);
        if (a + 1 < CH) {
            __syncthreads();
            dma_tile<true>(vbuf, V + (a + 1) * hstride, qt * BN, BN, T, wave, lane);
            wait_vm();
        }
    }

    // row sums l_b: the four lanes of a row, then the two key halves via LDS
#pragma unroll
    for (int s = 0; s < CH; ++s) {
        float l = l_run[s];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (g4 == 0) gnx[(kh * CH + s) * BM + io] = l;
    }
    __syncthreads();
    if (tid < CH * BM) {
        const int s = tid / BM, row = tid % BM;
        al[s * BM + row] = 1.0f / (gnx[(0 * CH + s) * BM + row] + gnx[(1 * CH + s) * BM + row]);
    }
    __syncthreads();

    // O^a = sum_b w_ab U_{b,a} / l_b  (rows 16rw + 4g4 + r)
    f32x4 acc[CH][D / 32];
    {
        float il[CH][4];
#pragma unroll
        for (int s = 0; s < CH; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) il[s][r] = al[s * BM + 16 * rw + 4 * g4 + r];
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o = 0.f;
#pragma unroll
                    for (int s = 0; s < CH; ++s) o = __builtin_fmaf(w_s[a * CH + s] * il[s][r], U[s][a][nb][r], o);
                    acc[a][nb][r] = o;
                }
    }

    // ---------------- epilogue: GroupNorm over d, head factor, store -------
    float mu[CH][4];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sum = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) sum += acc[a][nb][r];
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            sum += __shfl_xor(sum, 8);
            if (l16 == 0) gnx[(kh * CH + a) * BM + 16 * rw + 4 * g4 + r] = sum;
        }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rw + 4 * g4 + r;
            mu[a][r] = (gnx[(0 * CH + a) * BM + row] + gnx[(1 * CH + a) * BM + row]) * (1.0f / D);
        }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v2s = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
                const float dl = acc[a][nb][r] - mu[a][r];
                v2s = __builtin_fmaf(dl, dl, v2s);
            }
            v2s += __shfl_xor(v2s, 1);
            v2s += __shfl_xor(v2s, 2);
            v2s += __shfl_xor(v2s, 4);
            v2s += __shfl_xor(v2s, 8);
            if (l16 == 0) gnx[(kh * CH + a) * BM + 16 * rw + 4 * g4 + r] = v2s;
        }
    __syncthreads();
    bf16_t *O = reinterpret_cast<bf16_t *>(p.out);
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        const int h = h0 + a;
        const float *gw = p.gn_w + (size_t)h * D;
        const float *gb = p.gn_b + (size_t)h * D;
        const float hf = head_factor(p, h);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rowt = 16 * rw + 4 * g4 + r;
            const float var = (gnx[(0 * CH + a) * BM + rowt] + gnx[(1 * CH + a) * BM + rowt]) * (1.0f / D);
            const float rstd = 1.0f / __builtin_sqrtf(var + p.eps);
            const int row = i0 + rowt;
            if (row < T) {
                bf16_t *dst = O + ((size_t)b * p.H + h) * hstride + (size_t)row * D;
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb) {
                    const int col = dbase + 16 * nb + l16;
                    const float y = ((acc[a][nb][r] - mu[a][r]) * rstd * gw[col] + gb[col]) * hf;
                    dst[col] = (bf16_t)y;
                }
            }
        }
    }
}

template <int D, int CH, int CQ, int CK, bool EXACT>
hipError_t launch(const Params &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_v3<D, CH, CQ, CK, EXACT>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p);
    return hipGetLastError();
}

}  // namespace v3
}  // namespace mta
