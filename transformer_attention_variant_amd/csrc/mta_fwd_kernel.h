// mta_fwd_kernel.h — the fused Multi-Token Attention forward kernel for gfx950.
//
// Operation (page "Multi-Token Attention — Paper Graph", section 3.4):
//   S = Q K^T / sqrt(d)                               ("Standard Multi-Head Attention")
//   kq PRE : L = Mask_-inf(Conv2d_theta(Mask_0(S)))  (two-pass masking, "Key-Query
//            Convolution"), P = softmax(L)
//            or, exact form, L = Mask_-inf(Eq. 4 with its indicator 1{i >= j-j'})
//            on the unmasked S: a tap counts iff its key is not in the future of
//            the output query (p.exact)
//   kq POST: P = Mask_0(Conv2d_theta(softmax(Mask_-inf(S))))   (post-softmax variant)
//   head mix PRE (logits) or POST (probabilities), Eq. 7, groups of c_h heads
//   O = P V per head, then GroupNorm over d x depth scale.
//
// One workgroup (4 waves) owns (batch b, head group g, 64 query rows).  It never
// writes a T x T map: pass 1 walks the causal key tiles to get each row's
// softmax statistics of the map that enters the softmax; pass 2 walks them again,
// forms probabilities, mixes heads in registers and accumulates P V on the
// matrix cores; the epilogue normalises and stores.
//
// Per key tile and head:
//   * the logit tile with its halo — 16 rows above the tile (c_q-1 <= 15 of
//     them are read) and ceil(c_k/2)-1 / floor(c_k/2) key columns left/right —
//     is computed with MFMA (S^T = K Q^T, fp32 accumulate) and stored to LDS
//     in fp32, already scaled by log2(e)/sqrt(d) and with Mask_0 applied;
//   * each lane computes 16 consecutive outputs of one row with a register-
//     blocked stencil (c_q x c_k FMAs per output, kernel weights uniform);
//   * the 16 outputs of a lane are exactly the A-operand slots of the P V
//     MFMA for that row (16x16x32 bf16 or 16x16x4 f32), so probabilities go
//     from the stencil to the matrix cores without another LDS round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mta {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;            // query rows per workgroup
constexpr int BN = 64;            // keys per key tile (== BM: tile kt == qt is the diagonal)
constexpr int HALO = 16;          // logit-tile rows above the query tile
constexpr int EXT_R = HALO + BM;  // logit-tile rows
constexpr int NT = 256;           // threads per workgroup (4 waves of 64)
constexpr int MAX_CQ = 16;        // c_q - 1 <= HALO - 1
constexpr int MAX_CK = 31;        // keeps the logit tile within 96 columns
constexpr float NEG_INF = -__builtin_inff();

struct Params {
    const void *q, *k, *v;
    const float *theta;   // [H][c_q][c_k]
    const float *wmix;    // [H/c_h][c_h][c_h]
    const float *gn_w, *gn_b;
    const float *gate;    // [H] per-head gate logits, or null
    void *out;
    int H, T, c_q, c_k, G, units, n_qt;
    int head_pre;         // head mix before the softmax
    int exact;            // kq before the softmax with Eq. 4's exact indicator
    int ncb;              // 16-wide column blocks of the logit tile
    int pitch;            // floats per logit-tile row in LDS
    int hl;               // left key halo = ceil(c_k/2) - 1
    int nbuf;             // logit-tile buffers in LDS (c_h when every head's tile is needed at once)
    int npair;            // head-split kernel, groups of c_h >= 4 heads: source head pairs per group (c_h / 2)
    float sc;             // log2(e) / sqrt(d)
    float eps, depth_scale;
};

// Output factor of head h: depth_scale * sigmoid(gate[h]) with a gate
// ("Group Normalization with Sigmoid Gating"), depth_scale alone without.
__device__ inline float head_factor(const Params &p, int h)
{
    if (!p.gate) return p.depth_scale;
    return p.depth_scale / (1.0f + __expf(-p.gate[h]));
}

// ---------------------------------------------------------------------------
// LDS layout (floats unless noted), sized on the host by lds_bytes():
//   sbuf  : nbuf x EXT_R x pitch      logit / probability tiles
//   stats : 2 x c_h x EXT_R           row max (log2 domain) and 1/sum
//   theta : c_h x c_q x ckp           the group's key-query kernels, rows padded to 4
//   w     : c_h x c_h                 the group's mixing matrix (padded to 4)
//   vbuf  : bf16: D x VP_BF16 bf16    V tile transposed  (Vt[dcol][key])
//           f32 : BN x (D + 4)        V tile row-major    (V[key][dcol])
constexpr int VP_BF16 = BN + 8;

template <typename DT, int D>
__host__ __device__ constexpr int vbuf_bytes()
{
    return sizeof(DT) == 2 ? D * VP_BF16 * 2 : BN * (D + 4) * 4;
}

// ---------------------------------------------------------------------------
// Logit block: 16 keys x 16 queries, D^T[key m][query n] = sum_d K[m][d] Q[n][d].
// MFMA lane layout (16x16 shapes): A row = lane%16, B column = lane%16, output
// lane holds column n = lane%16 and rows m = 4*(lane/16) + r.  The contraction
// index is permuted so that lane group lane/16 reads a contiguous quarter of d
// (same permutation on both operands, so the dot product is unchanged).
template <int D>
struct QFrag {
    bf16x8 x[D / 32];
};

template <int D>
__device__ inline void load_frag(QFrag<D> &f, const bf16_t *base, int row, int T, int lane)
{
    const int dq = (lane >> 4) * (D / 4);
    if ((unsigned)row < (unsigned)T) {
        const bf16x8 *p = reinterpret_cast<const bf16x8 *>(base + (size_t)row * D + dq);
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
__device__ inline f32x4 qk_mfma(const QFrag<D> &kf, const QFrag<D> &qf)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.x[t], qf.x[t], acc, 0, 0, 0);
    return acc;
}

template <int D>
struct QFrag32 {
    f32x4 x[D / 16];
};

template <int D>
__device__ inline void load_frag(QFrag32<D> &f, const float *base, int row, int T, int lane)
{
    const int dq = (lane >> 4) * (D / 4);
    if ((unsigned)row < (unsigned)T) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(base + (size_t)row * D + dq);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) f.x[t] = p[t];
    } else {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) f.x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

template <int D>
__device__ inline f32x4 qk_mfma(const QFrag32<D> &kf, const QFrag32<D> &qf)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.x[t][e], qf.x[t][e], acc, 0, 0, 0);
    return acc;
}

template <typename DT, int D>
struct FragOf {
    typedef QFrag<D> type;
};
template <int D>
struct FragOf<float, D> {
    typedef QFrag32<D> type;
};

// ---------------------------------------------------------------------------
// Store one 16x16 logit block into the LDS tile.  Tile row rho <-> query
// i0 - HALO + rho, tile column e <-> key j0 - hl + e.  Mode RAW writes
// x = S*log2(e)/sqrt(d) where 0 <= key <= kmax and 0 <= query < T, 0 elsewhere:
// kmax = query gives Mask_0 and the zero padding of the convolution; with
// `exact` kmax = T-1 keeps the future logits (Eq. 4's indicator is then applied
// per output row by the stencil).  Mode PROB writes the probability
// exp2(x - m_rho) / l_rho where the key is causal instead.
enum TileMode { RAW = 0, PROB = 1 };

template <int MODE>
__device__ inline void store_block(float *buf, int pitch, int rb, int cb, f32x4 acc, int i0, int j0,
                                   int hl, int T, float sc, const float *st_m, const float *st_il,
                                   int exact, int lane)
{
    const int rho = rb * 16 + (lane & 15);
    const int e0 = cb * 16 + 4 * (lane >> 4);
    const int qi = i0 - HALO + rho;
    const int kmax = (MODE == RAW && exact) ? T - 1 : qi;
    float m = 0.f, il = 0.f;
    if (MODE == PROB) {
        m = st_m[rho];
        il = st_il[rho];
    }
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int kj = j0 - hl + e0 + r;
        const bool ok = (kj >= 0) && (kj <= kmax) && (qi >= 0) && (qi < T);
        float x = acc[r] * sc;
        if (MODE == PROB) x = __builtin_amdgcn_exp2f(x - m) * il;
        o[r] = ok ? x : 0.f;
    }
    *reinterpret_cast<f32x4 *>(buf + rho * pitch + e0) = o;
}

// Compute the whole logit tile of one head into `buf`.  Wave w owns tile rows
// [HALO + 16w, HALO + 16w + 16) (its own query rows) for every column block;
// the HALO block (rows above the query tile) is shared out by column block.
template <typename DT, int D, int MODE>
__device__ inline void logit_tile(float *buf, const Params &p, const DT *qh, const DT *kh, int i0,
                                  int j0, const float *st_m, const float *st_il, int wave, int lane)
{
    typedef typename FragOf<DT, D>::type Frag;
    Frag qf, kf;
    const int kcol = j0 - p.hl + (lane & 15);
    // own rows
    load_frag<D>(qf, qh, i0 + wave * 16 + (lane & 15), p.T, lane);
    for (int cb = 0; cb < p.ncb; ++cb) {
        load_frag<D>(kf, kh, kcol + cb * 16, p.T, lane);
        const f32x4 acc = qk_mfma<D>(kf, qf);
        store_block<MODE>(buf, p.pitch, 1 + wave, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, p.exact,
                          lane);
    }
    // halo rows, only if the kernel reaches back (c_q > 1)
    if (p.c_q > 1) {
        load_frag<D>(qf, qh, i0 - HALO + (lane & 15), p.T, lane);
        for (int cb = wave; cb < p.ncb; cb += 4) {
            load_frag<D>(kf, kh, kcol + cb * 16, p.T, lane);
            const f32x4 acc = qk_mfma<D>(kf, qf);
            store_block<MODE>(buf, p.pitch, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, p.exact,
                              lane);
        }
    }
}

// ---------------------------------------------------------------------------
// Key-query stencil: 16 consecutive outputs of one row.
//   out[o] = sum_{i'} sum_{jj} theta[i'][jj] * X[rho - i'][jb + o + c_k - 1 - jj]
// (tile column jb + o + c_k - 1 - jj holds key j - j' for output key j and
// j' = jj - floor(c_k/2), since the tile starts hl = ceil(c_k/2)-1 keys left).
// The kernel weights come from LDS (`th`, rows of `ckp` floats, ckp a multiple
// of 4), read as broadcast vectors.  Window entries t > tlim (tile column
// jb + t) are taken as 0: with Eq. 4's indicator tlim is the last column whose
// key is not in the future of this lane's output query; the tile already holds
// 0 there in the two-pass form, which passes tlim >= the window length.
template <int CQ, int CK>
__device__ inline void stencil16(const float *buf, int pitch, int rho, int jb, const float *th,
                                 int, int, int, int tlim, float out[16])
{
    constexpr int NW = 16 + CK - 1;
    constexpr int NW4 = (NW + 3) / 4;
    constexpr int CK4 = (CK + 3) / 4;
#pragma unroll
    for (int o = 0; o < 16; ++o) out[o] = 0.f;
    // the query-offset loop stays rolled: one window of 16 + c_k - 1 values and
    // one kernel row live at a time
#pragma unroll 1
    for (int ip = 0; ip < CQ; ++ip) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(buf + (rho - ip) * pitch + jb);
        const f32x4 *trow = reinterpret_cast<const f32x4 *>(th + ip * (CK4 * 4));
        float win[NW4 * 4], tw[CK4 * 4];
#pragma unroll
        for (int t = 0; t < NW4; ++t) {
            const f32x4 x = row[t];
            win[4 * t + 0] = x[0];
            win[4 * t + 1] = x[1];
            win[4 * t + 2] = x[2];
            win[4 * t + 3] = x[3];
        }
        if (tlim < NW - 1) {
#pragma unroll
            for (int t = 0; t < NW; ++t) win[t] = (t <= tlim) ? win[t] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < CK4; ++t) {
            const f32x4 x = trow[t];
            tw[4 * t + 0] = x[0];
            tw[4 * t + 1] = x[1];
            tw[4 * t + 2] = x[2];
            tw[4 * t + 3] = x[3];
        }
#pragma unroll
        for (int jj = 0; jj < CK; ++jj) {
#pragma unroll
            for (int o = 0; o < 16; ++o) out[o] = __builtin_fmaf(tw[jj], win[o + CK - 1 - jj], out[o]);
        }
    }
}

// Runtime-sized variant (any c_q <= 16, c_k <= MAX_CK): same sum.  Per query
// offset the lane loads its window of 16 + c_k - 1 values into registers once;
// the taps are unrolled to MAX_CK with a uniform guard, walking the window with
// compile-time register indices (tap m multiplies window entry o + m by the
// kernel weight of column c_k - 1 - m, read from LDS as a broadcast).
template <>
__device__ inline void stencil16<0, 0>(const float *buf, int pitch, int rho, int jb, const float *th,
                                       int cq, int ck, int ckp, int tlim, float out[16])
{
    constexpr int NWMAX = 16 + MAX_CK - 1;
    constexpr int NW4MAX = (NWMAX + 3) / 4;
    const int nw = 16 + ck - 1;
    const int nw4 = (nw + 3) / 4;
#pragma unroll
    for (int o = 0; o < 16; ++o) out[o] = 0.f;
    for (int ip = 0; ip < cq; ++ip) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(buf + (rho - ip) * pitch + jb);
        float win[NW4MAX * 4];
#pragma unroll
        for (int t = 0; t < NW4MAX; ++t) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (t < nw4) x = row[t];
            win[4 * t + 0] = x[0];
            win[4 * t + 1] = x[1];
            win[4 * t + 2] = x[2];
            win[4 * t + 3] = x[3];
        }
        if (tlim < nw - 1) {
#pragma unroll
            for (int t = 0; t < NWMAX; ++t) win[t] = (t <= tlim) ? win[t] : 0.f;
        }
        const float *trow = th + ip * ckp;
#pragma unroll
        for (int m = 0; m < MAX_CK; ++m) {
            if (m < ck) {
                const float tv = trow[ck - 1 - m];
#pragma unroll
                for (int o = 0; o < 16; ++o) out[o] = __builtin_fmaf(tv, win[o + m], out[o]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Online softmax statistics of one lane's 16 values (log2 domain).  Only
// entries with key <= query count; the lane's partial (m, l) is merged with the
// other lanes of the row once, at the end of pass 1.
__device__ inline void stats_update(const float x[16], int key0, int query, float &m, float &l)
{
    float tmax = NEG_INF;
#pragma unroll
    for (int o = 0; o < 16; ++o)
        if (key0 + o <= query) tmax = fmaxf(tmax, x[o]);
    const float mn = fmaxf(m, tmax);
    if (mn == NEG_INF) return;  // nothing causal seen yet
    float s = (m == NEG_INF) ? 0.f : l * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int o = 0; o < 16; ++o)
        if (key0 + o <= query) s += __builtin_amdgcn_exp2f(x[o] - mn);
    m = mn;
    l = s;
}

// Merge the partial statistics of the four lanes that share a row (lane,
// lane^16, lane^32, lane^48) with wave shuffles; returns max and 1/sum.
__device__ inline void stats_merge(float m, float l, float &M, float &IL)
{
    float mx = fmaxf(m, __shfl_xor(m, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float s = (m == NEG_INF) ? 0.f : l * __builtin_amdgcn_exp2f(m - mx);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    M = mx;
    IL = 1.0f / s;
}

// ---------------------------------------------------------------------------
// V tile for one head into LDS.
template <int D>
__device__ inline void load_v_tile(bf16_t *vb, const bf16_t *vh, int j0, int T, int tid)
{
    // thread -> key (tid % 64), 8 channels per step: consecutive lanes write
    // consecutive keys of one transposed row.
    const int key = tid & 63;
    const int kj = j0 + key;
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
        const int c0 = ((tid >> 6) + 4 * it) * 8;
        bf16x8 x;
        if (kj < T) {
            x = *reinterpret_cast<const bf16x8 *>(vh + (size_t)kj * D + c0);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (bf16_t)0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[(c0 + e) * VP_BF16 + key] = x[e];
    }
}

template <int D>
__device__ inline void load_v_tile(float *vb, const float *vh, int j0, int T, int tid)
{
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < BN * C4; idx += NT) {
        const int key = idx / C4, c0 = (idx % C4) * 4;
        const int kj = j0 + key;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (kj < T) x = *reinterpret_cast<const f32x4 *>(vh + (size_t)kj * D + c0);
        *reinterpret_cast<f32x4 *>(vb + key * (D + 4) + c0) = x;
    }
}

// O[16 rows x D] += P(16 rows x 64 keys) V(64 keys x D) for one head.
// Lane holds P for row lane%16, keys 16*(lane/16) + [0,16).
template <int D>
__device__ inline void pv_mfma(f32x4 (&acc)[D / 16], const float pr[16], const bf16_t *vb, int lane)
{
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (bf16_t)pr[8 * c + e];
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
            const bf16x8 bv =
                *reinterpret_cast<const bf16x8 *>(vb + (nb * 16 + n) * VP_BF16 + kg * 16 + 8 * c);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[nb], 0, 0, 0);
        }
    }
}

template <int D>
__device__ inline void pv_mfma(f32x4 (&acc)[D / 16], const float pr[16], const float *vb, int lane)
{
    const int n = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
            const float bv = vb[(kg * 16 + t) * (D + 4) + nb * 16 + n];
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[t], bv, acc[nb], 0, 0, 0);
        }
    }
}

template <typename DT>
__device__ inline DT cvt_out(float x)
{
    return (DT)x;
}

// ---------------------------------------------------------------------------
// In-register head mix of one lane's 16 values over the c_h heads of a group:
// x[a] <- sum_b w[a][b] x[b]  (Eq. 7 on probabilities, or its pre-softmax
// form on logits).  w from LDS, [c_h][c_h].
template <int CH>
__device__ inline void head_mix16(float (&x)[CH][16], const float *w)
{
#pragma unroll
    for (int o = 0; o < 16; ++o) {
        float y[CH];
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            float s = 0.f;
#pragma unroll
            for (int bb = 0; bb < CH; ++bb) s = __builtin_fmaf(w[a * CH + bb], x[bb][o], s);
            y[a] = s;
        }
#pragma unroll
        for (int a = 0; a < CH; ++a) x[a][o] = y[a];
    }
}

// ---------------------------------------------------------------------------
template <typename DT, int D, int CH, int CQ, int CK, bool KQ_POST, bool HPRE>
__global__ void __launch_bounds__(NT) mta_fwd_kernel(Params p)
{
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;  // longest rows first
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;

    const int cq = CQ ? CQ : p.c_q;
    const int ck = CK ? CK : p.c_k;
    const int ckp = (ck + 3) & ~3;

    // LDS carve-up (all offsets multiples of 16 bytes)
    float *sbuf = lds;
    float *st_m = sbuf + p.nbuf * EXT_R * p.pitch;
    float *st_il = st_m + CH * EXT_R;
    float *th_s = st_il + CH * EXT_R;                   // [CH][cq][ckp]
    float *w_s = th_s + ((CH * cq * ckp + 3) & ~3);     // [CH][CH]
    DT *vbuf = reinterpret_cast<DT *>(w_s + ((CH * CH + 3) & ~3));

    const size_t hstride = (size_t)T * D;
    const DT *Q = reinterpret_cast<const DT *>(p.q);
    const DT *K = reinterpret_cast<const DT *>(p.k);
    const DT *V = reinterpret_cast<const DT *>(p.v);
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;

    // kernel weights of the group's heads and the group's mixing matrix
    for (int i = tid; i < CH * cq * ckp; i += NT) {
        const int a = i / (cq * ckp), r = (i / ckp) % cq, c = i % ckp;
        th_s[i] = c < ck ? p.theta[((size_t)(h0 + a) * cq + r) * ck + c] : 0.f;
    }
    for (int i = tid; i < CH * CH; i += NT) w_s[i] = p.wmix[(size_t)g * CH * CH + i];

    // this lane's output row and key columns
    const int io = wave * 16 + (lane & 15);  // row within the query tile
    const int jb = 16 * (lane >> 4);         // first of 16 key columns within the key tile
    const int qabs = i0 + io;
    const int rho = HALO + io;                // logit-tile row of this output row
    const int qhalo = i0 - HALO + (lane & 15); // query of halo row lane%16 (wave 0)

    // ---------------- pass 1: row statistics ------------------------------
    float m_c[CH], l_c[CH], m_h[CH], l_h[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        m_c[a] = NEG_INF; l_c[a] = 0.f; m_h[a] = NEG_INF; l_h[a] = 0.f;
    }

    constexpr int NOLIM = 1 << 30;
    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        const int key0 = j0 + jb;
        // last window column whose key is not in this row's future (exact form)
        const int tlim = p.exact ? qabs - (j0 - p.hl + jb) : NOLIM;
        if (!KQ_POST) {
            if (HPRE) {
                float c[CH][16];
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    __syncthreads();
                    logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride,
                                           i0, j0, nullptr, nullptr, wave, lane);
                    __syncthreads();
                    stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + a * cq * ckp, cq, ck, ckp, tlim, c[a]);
                }
                head_mix16<CH>(c, w_s);
#pragma unroll
                for (int a = 0; a < CH; ++a) stats_update(c[a], key0, qabs, m_c[a], l_c[a]);
            } else {
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    float c[16];
                    __syncthreads();
                    logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride,
                                           i0, j0, nullptr, nullptr, wave, lane);
                    __syncthreads();
                    stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + a * cq * ckp, cq, ck, ckp, tlim, c);
                    stats_update(c, key0, qabs, m_c[a], l_c[a]);
                }
            }
        } else {
            // statistics of the (head-mixed, if HPRE) logits for the tile's rows
            // and for the rows above it, over the tile's own keys
            if (HPRE) {
                __syncthreads();
                for (int a = 0; a < CH; ++a)
                    logit_tile<DT, D, RAW>(sbuf + a * EXT_R * p.pitch, p, Q + base0 + a * hstride,
                                           K + base0 + a * hstride, i0, j0, nullptr, nullptr, wave, lane);
                __syncthreads();
                float xc[CH][16];
#pragma unroll
                for (int a = 0; a < CH; ++a)
#pragma unroll
                    for (int o = 0; o < 16; ++o) xc[a][o] = sbuf[a * EXT_R * p.pitch + rho * p.pitch + p.hl + jb + o];
                head_mix16<CH>(xc, w_s);
#pragma unroll
                for (int a = 0; a < CH; ++a) stats_update(xc[a], key0, qabs, m_c[a], l_c[a]);
                if (wave == 0) {
#pragma unroll
                    for (int a = 0; a < CH; ++a)
#pragma unroll
                        for (int o = 0; o < 16; ++o)
                            xc[a][o] = sbuf[a * EXT_R * p.pitch + (lane & 15) * p.pitch + p.hl + jb + o];
                    head_mix16<CH>(xc, w_s);
#pragma unroll
                    for (int a = 0; a < CH; ++a) stats_update(xc[a], key0, qhalo, m_h[a], l_h[a]);
                }
            } else {
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    __syncthreads();
                    logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride,
                                           i0, j0, nullptr, nullptr, wave, lane);
                    __syncthreads();
                    float x[16];
#pragma unroll
                    for (int o = 0; o < 16; ++o) x[o] = sbuf[rho * p.pitch + p.hl + jb + o];
                    stats_update(x, key0, qabs, m_c[a], l_c[a]);
                    if (wave == 0) {
#pragma unroll
                        for (int o = 0; o < 16; ++o) x[o] = sbuf[(lane & 15) * p.pitch + p.hl + jb + o];
                        stats_update(x, key0, qhalo, m_h[a], l_h[a]);
                    }
                }
            }
        }
    }

    float M[CH], IL[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) stats_merge(m_c[a], l_c[a], M[a], IL[a]);
    if (KQ_POST) {
        float Mh[CH], ILh[CH];
#pragma unroll
        for (int a = 0; a < CH; ++a) stats_merge(m_h[a], l_h[a], Mh[a], ILh[a]);
        if (lane < 16) {
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                st_m[a * EXT_R + rho] = M[a];
                st_il[a * EXT_R + rho] = IL[a];
                if (wave == 0) {
                    // rows above the sequence start have no causal entry: zero padding
                    const bool live = qhalo >= 0;
                    st_m[a * EXT_R + lane] = live ? Mh[a] : 0.f;
                    st_il[a * EXT_R + lane] = live ? ILh[a] : 0.f;
                }
            }
        }
        __syncthreads();
    }

    // ---------------- pass 2: probabilities, head mix, P V -----------------
    f32x4 acc[CH][D / 16];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) acc[a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
        const int key0 = j0 + jb;
        const int tlim = p.exact ? qabs - (j0 - p.hl + jb) : NOLIM;
        float pr[CH][16];
        if (!KQ_POST) {
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                __syncthreads();
                logit_tile<DT, D, RAW>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride, i0,
                                       j0, nullptr, nullptr, wave, lane);
                __syncthreads();
                stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + a * cq * ckp, cq, ck, ckp, tlim, pr[a]);
                if (!HPRE) {
#pragma unroll
                    for (int o = 0; o < 16; ++o)
                        pr[a][o] = (key0 + o <= qabs) ? __builtin_amdgcn_exp2f(pr[a][o] - M[a]) * IL[a] : 0.f;
                }
            }
            if (HPRE) {
                head_mix16<CH>(pr, w_s);
#pragma unroll
                for (int a = 0; a < CH; ++a)
#pragma unroll
                    for (int o = 0; o < 16; ++o)
                        pr[a][o] = (key0 + o <= qabs) ? __builtin_amdgcn_exp2f(pr[a][o] - M[a]) * IL[a] : 0.f;
            }
        } else if (!HPRE) {
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                __syncthreads();
                logit_tile<DT, D, PROB>(sbuf, p, Q + base0 + a * hstride, K + base0 + a * hstride, i0,
                                        j0, st_m + a * EXT_R, st_il + a * EXT_R, wave, lane);
                __syncthreads();
                stencil16<CQ, CK>(sbuf, p.pitch, rho, jb, th_s + a * cq * ckp, cq, ck, ckp, NOLIM, pr[a]);
#pragma unroll
                for (int o = 0; o < 16; ++o) pr[a][o] = (key0 + o <= qabs) ? pr[a][o] : 0.f;  // Mask_0
            }
        } else {
            // head mix on the logits of the whole tile, then probabilities
            __syncthreads();
            for (int a = 0; a < CH; ++a)
                logit_tile<DT, D, RAW>(sbuf + a * EXT_R * p.pitch, p, Q + base0 + a * hstride,
                                       K + base0 + a * hstride, i0, j0, nullptr, nullptr, wave, lane);
            __syncthreads();
            const int r_lo = HALO - (cq - 1);
            const int ncol = p.ncb * 16;
            for (int idx = tid; idx < (EXT_R - r_lo) * ncol; idx += NT) {
                const int r = r_lo + idx / ncol, e = idx % ncol;
                const int qi = i0 - HALO + r, kj = j0 - p.hl + e;
                const bool ok = (kj >= 0) && (kj <= qi) && (qi < T);
                float x[CH];
#pragma unroll
                for (int a = 0; a < CH; ++a) x[a] = sbuf[a * EXT_R * p.pitch + r * p.pitch + e];
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    float s = 0.f;
#pragma unroll
                    for (int bb = 0; bb < CH; ++bb) s = __builtin_fmaf(w_s[a * CH + bb], x[bb], s);
                    const float pv = __builtin_amdgcn_exp2f(s - st_m[a * EXT_R + r]) * st_il[a * EXT_R + r];
                    sbuf[a * EXT_R * p.pitch + r * p.pitch + e] = ok ? pv : 0.f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int a = 0; a < CH; ++a) {
                stencil16<CQ, CK>(sbuf + a * EXT_R * p.pitch, p.pitch, rho, jb, th_s + a * cq * ckp, cq,
                                  ck, ckp, NOLIM, pr[a]);
#pragma unroll
                for (int o = 0; o < 16; ++o) pr[a][o] = (key0 + o <= qabs) ? pr[a][o] : 0.f;  // Mask_0
            }
        }

        // head mix after the softmax (Eq. 7)
        if (!HPRE) head_mix16<CH>(pr, w_s);

        // P V, one head at a time through the V tile buffer
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            __syncthreads();
            load_v_tile<D>(vbuf, V + base0 + a * hstride, j0, T, tid);
            __syncthreads();
            pv_mfma<D>(acc[a], pr[a], vbuf, lane);
        }
    }

    // ---------------- epilogue: GroupNorm over d, depth scale, store -------
    // acc[a][nb][r] = O[row 16*wave + 4*(lane/16) + r][col 16*nb + lane%16]
    DT *O = reinterpret_cast<DT *>(p.out);
    const int n = lane & 15;
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        const int h = h0 + a;
        const float *gw = p.gn_w + (size_t)h * D;
        const float *gb = p.gn_b + (size_t)h * D;
        const float hf = head_factor(p, h);
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

}  // namespace mta
