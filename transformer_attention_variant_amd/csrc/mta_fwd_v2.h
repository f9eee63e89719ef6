// mta_fwd_v2.h — pipelined 8-wave MTA forward for bf16 (the large workloads).
//
// Same operation and two-pass structure as mta_fwd_kernel.h (page "Multi-Token
// Attention — Paper Graph", section 3.4: logits, key-query convolution with
// two-pass masking or after the softmax, softmax, head mixing after the softmax
// (Eq. 7), A·V, GroupNorm x depth scale), organised for latency hiding on gfx950:
//
//  * 8 waves per workgroup, two per SIMD.  Wave w = (row block rw = w%4, half
//    kh = w/4): in the stencil it owns the 16 query rows 16rw.. of the tile and
//    the 32 keys 32kh.. of each key tile (a lane: one row, 8 keys); in P·V it
//    owns the same 16 rows and the d-columns [kh*d/2, (kh+1)*d/2).
//  * The work is a sequence of phases, one per (key tile kt, head a).  A phase
//    has an MFMA part (logit tile of (kt, a) from the Q and K tiles in LDS, and
//    P·V of tile kt-1 for head a) and a stencil part (convolution, softmax
//    statistics or probabilities).  Two barriers per phase.
//  * Global loads of the next phase's Q, K and V tiles are issued at the start
//    of the (long) stencil part into registers and written to LDS at its end,
//    so their latency hides behind the stencil.
//  * Probabilities of a key tile, mixed across the head group, are exchanged
//    through LDS in the MFMA A-operand layout; each wave then multiplies the
//    full 64-key tile by its half of V.
#pragma once

#include "mta_fwd_kernel.h"

namespace mta {
namespace v2 {

constexpr int NW = 8;
constexpr int NT = 64 * NW;
// LDS pitches (bf16 elements) of the row-major Q, K and V tiles.  A row of
// D + 16 elements is an even number of 16-byte chunks plus two, so the 16 rows
// read by one 16-lane group land on distinct bank groups; with frag_base below
// (lane groups 0/1 and 2/3 an odd number of chunks apart) the 32 lanes served
// together by one ds_read_b128 never share a bank, and the transposing V reads
// are conflict-free as well.
template <int D>
__host__ __device__ constexpr int kpitch() { return D + 16; }
template <int D>
__host__ __device__ constexpr int vpitch() { return D + 16; }

// The logit product of a 16x16 block is a sum over d; lane group g4 supplies
// the 16-byte chunk fc + 2t (fc = frag_base / 8) of its Q or K row to MFMA
// step t.  Any assignment that covers every chunk once works when Q and K use
// the same one.
template <int D>
__device__ inline int frag_base(int lane)
{
    const int g4 = lane >> 4;
    return 8 * ((g4 & 1) + (D / 16) * (g4 >> 1));
}

struct Layout {
    int s_off, k_off, q_off, v_off, p_off, st_off, xs_off, th_off, w_off, gn_off, tf_off, cr_off, total;
};

// Centre-tap correction plane of the matrix-core stencil before the softmax:
// fp16 [row of the query tile][key of the key tile], pitch CRP2 (34 banks per
// row: the stencil's 8-byte reads of 16 rows never share a bank), followed by
// one flag per own-row logit block, [row block][column block] (CRF column
// blocks), saying whether the block wrote corrections.
constexpr int CRP2 = 68;
constexpr int CRF = 8;

// fp16 pitch of the logit tile of the matrix-core stencil: a multiple of 8
// elements whose 16-byte chunk count is 2 mod 4, so that the stencil's
// ds_read_b128 (16 rows x 2 adjacent chunks per pass) never shares a bank.
__host__ __device__ inline int pitch_hl(int ncb) { return (ncb & 1) ? ncb * 16 : ncb * 16 + 16; }

// post: the convolution follows the softmax (pass 1 then keeps raw fp32
// logits for the statistics, also with the matrix-core stencil)
__host__ __device__ inline Layout layout(int D, int CH, int cq, int ck, int ncb, int pitch, bool ms, bool post)
{
    Layout L;
    int o = 0;
    const int KP = D + 16;
    const int sb32 = EXT_R * pitch * 4, sb16 = EXT_R * pitch_hl(ncb) * 2;
    const int sb = (ms && !post) ? sb16 : (sb32 > sb16 ? sb32 : sb16);
    L.s_off = o;  o += sb;                                  // logit / probability tile (fp32, or fp16)
    L.k_off = o;  o += ncb * 16 * KP * 2;                   // K tile with key halo (bf16)
    L.q_off = o;  o += EXT_R * KP * 2;                      // Q tile with the 16 rows above (bf16)
    L.v_off = o;  o += BN * KP * 2;                         // V tile, row-major (bf16)
    L.p_off = o;  o += CH * 4 * 2 * 64 * 16;                // mixed probabilities [a][rw][chunk][lane] x 8 bf16
    L.st_off = o; o += 2 * CH * EXT_R * 4;                  // final row statistics m, 1/l per tile row
    L.xs_off = o; o += 2 * CH * EXT_R * 2 * 4;              // per-half partial statistics
    L.th_off = o; o += ((CH * cq * ((ck + 3) & ~3) + 3) & ~3) * 4;
    L.w_off = o;  o += ((CH * CH + 3) & ~3) * 4;
    L.gn_off = o; o += 2 * CH * BM * 4;                     // GroupNorm partial sums per d half
    L.tf_off = o; o += ms ? CH * cq * 64 * 16 : 0;          // banded kernel matrices as MFMA A operands (fp16)
    L.cr_off = o; o += (ms && !post) ? BM * CRP2 * 2 + 4 * CRF * 4 : 0;  // centre-tap corrections, flags
    L.total = o;
    return L;
}

// ---------------------------------------------------------------------------
// Register prefetch of the next phase's tiles.
template <int D>
struct Pref {
    static constexpr int C8 = D / 8;                       // 16-byte chunks per row
    static constexpr int KL = (6 * 16 * C8 + NT - 1) / NT; // up to 96 key rows
    static constexpr int QL = (EXT_R * C8 + NT - 1) / NT;
    static constexpr int VL = (BN * C8 + NT - 1) / NT;
    bf16x8 k[KL], q[QL], v[VL];
};

__device__ inline bf16x8 zero8()
{
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16_t)0.0f;
    return z;
}

// K rows [j0 - hl, j0 - hl + 16*ncb) of one head (zero outside [0, T)).
template <int D>
__device__ inline void load_k(Pref<D> &r, const bf16_t *kh, int j0, int hl, int nrows, int T, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::KL; ++it) {
        const int idx = tid + it * NT;
        const int row = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        const int key = j0 - hl + row;
        r.k[it] = (row < nrows && key >= 0 && key < T)
                      ? *reinterpret_cast<const bf16x8 *>(kh + (size_t)key * D + 8 * c8)
                      : zero8();
    }
}

template <int D>
__device__ inline void store_k(const Pref<D> &r, bf16_t *kbuf, int nrows, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::KL; ++it) {
        const int idx = tid + it * NT;
        const int row = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        if (row < nrows) *reinterpret_cast<bf16x8 *>(kbuf + row * kpitch<D>() + 8 * c8) = r.k[it];
    }
}

// Q rows [i0 - HALO, i0 + BM) of one head.
template <int D>
__device__ inline void load_q(Pref<D> &r, const bf16_t *qh, int i0, int T, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::QL; ++it) {
        const int idx = tid + it * NT;
        const int row = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        const int qi = i0 - HALO + row;
        r.q[it] = (row < EXT_R && qi >= 0 && qi < T)
                      ? *reinterpret_cast<const bf16x8 *>(qh + (size_t)qi * D + 8 * c8)
                      : zero8();
    }
}

template <int D>
__device__ inline void store_q(const Pref<D> &r, bf16_t *qbuf, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::QL; ++it) {
        const int idx = tid + it * NT;
        const int row = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        if (row < EXT_R) *reinterpret_cast<bf16x8 *>(qbuf + row * kpitch<D>() + 8 * c8) = r.q[it];
    }
}

// V rows [j0, j0 + BN) of one head, stored row-major; the P.V product reads
// it with the transposing LDS load.
template <int D>
__device__ inline void load_v(Pref<D> &r, const bf16_t *vh, int j0, int T, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::VL; ++it) {
        const int idx = tid + it * NT;
        const int key = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        const int kj = j0 + key;
        r.v[it] = (key < BN && kj < T) ? *reinterpret_cast<const bf16x8 *>(vh + (size_t)kj * D + 8 * c8)
                                        : zero8();
    }
}

template <int D>
__device__ inline void store_v(const Pref<D> &r, bf16_t *vbuf, int tid)
{
#pragma unroll
    for (int it = 0; it < Pref<D>::VL; ++it) {
        const int idx = tid + it * NT;
        const int key = idx / Pref<D>::C8, c8 = idx % Pref<D>::C8;
        if (key < BN) *reinterpret_cast<bf16x8 *>(vbuf + key * vpitch<D>() + 8 * c8) = r.v[it];
    }
}

// Transposing LDS load (ds_read_b64_tr_b16): within each 16-lane group, element
// e = 0..3 of lane i is the (i mod 4)-th element of the 4-element row addressed
// by lane 4e + i/4.  With lane j addressing V[kb + j/4][d0 + 4(j%4)],
// lane i receives V[kb + e][d0 + i], e = 0..3: four consecutive keys of its
// own d column.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline s16x4 lds_read_tr4(const bf16_t *vbuf, int pitch, int kb, int d0, int j)
{
    const bf16_t *a = vbuf + (kb + (j >> 2)) * pitch + d0 + 4 * (j & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(a));
}

// ---------------------------------------------------------------------------
// Matrix-core stencil.  The key-query convolution of a 16-key output block is
// a banded (Toeplitz) product along keys, summed over the c_q query offsets:
//   C^T[m][n] = sum_{i'} sum_k Theta_{i'}[m][k] * X[row(n) - i'][w0 + k],
//   Theta_{i'}[m][k] = theta[i'][m + c_k - 1 - k] inside the band, else 0,
// for output key w0 + m (w0 = first column of the 32-column input window) and
// query row(n).  Both operands are rounded to fp16 (11 significant bits,
// magnitudes clamped to the fp16 range) and one product per kernel row
// accumulates in fp32 on the matrix cores.

typedef _Float16 f16_t;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// never inf, so a zero tap never meets an infinity
__device__ inline float f16_clamp(float x) { return __builtin_amdgcn_fmed3f(x, -65504.f, 65504.f); }

// Store a 16x16 logit block as fp16 (Mask_0 + zero padding applied; with
// `exact` only the zero padding, as in store_block); MODE PROB stores
// probabilities exp2(x - m_row) / l_row instead.
// With `cr` (before the softmax, own rows only): for a block holding a logit
// above 8 / |c00| in magnitude (log2 units; below it the fp16 rounding of the
// centre product stays under the bf16 rounding of the probabilities) the
// centre tap's correction c00 x - c00h fp16(x) of each stored logit (c00: the
// centre tap, c00h: its fp16 value in the banded matrices) goes to the
// correction plane at its output key, so that the stencil's centre product
// becomes exact there; the block's flag says whether it did.
template <int MODE>
__device__ inline void store_block_x(f16_t *x16, int ph, int rb, int cb, f32x4 acc, int i0, int j0, int hl, int T,
                                     float sc, const float *st_m, const float *st_il, int exact, int lane,
                                     f16_t *cr = nullptr, float c00 = 0.f, float c00h = 0.f)
{
    const int rho = rb * 16 + (lane & 15);
    const int e0 = cb * 16 + 4 * (lane >> 4);
    const int qi = i0 - HALO + rho;
    const bool ex = MODE == RAW && exact;
    const int kmax = ex ? T - 1 : qi;
    // block-uniform classification: every entry kept and inside [0, T), or not
    const int q_lo = i0 - HALO + rb * 16, k_lo = j0 - hl + cb * 16;
    const bool all_ok = (k_lo >= 0) && (k_lo + 15 <= (ex ? T - 1 : q_lo)) && (q_lo >= 0) && (q_lo + 15 < T);
    float m = 0.f, il = 0.f;
    if (MODE == PROB) {
        m = st_m[rho];
        il = st_il[rho];
    }
    float xv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x = acc[r] * sc;
        if (MODE == PROB) x = __builtin_amdgcn_exp2f(x - m) * il;
        if (!all_ok) {
            const int kj = j0 - hl + e0 + r;
            const bool ok = (kj >= 0) && (kj <= kmax) && (qi >= 0) && (qi < T);
            x = ok ? x : 0.f;
        }
        xv[r] = x;
    }
    const f16x4 h = {(f16_t)f16_clamp(xv[0]), (f16_t)f16_clamp(xv[1]), (f16_t)f16_clamp(xv[2]),
                     (f16_t)f16_clamp(xv[3])};
    *reinterpret_cast<f16x4 *>(x16 + rho * ph + e0) = h;
    if (MODE == RAW && cr && rb > 0) {
        const float big = fmaxf(fmaxf(fabsf(xv[0]), fabsf(xv[1])), fmaxf(fabsf(xv[2]), fabsf(xv[3])));
        const bool any = __builtin_amdgcn_ballot_w64(big * fabsf(c00) > 8.0f) != 0;  // wave-uniform
        if (any) {
            f16_t *crow = cr + (rho - HALO) * CRP2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = e0 + r - hl;  // output key of the entry
                if (o >= 0 && o < BN) crow[o] = (f16_t)__builtin_fmaf(c00, xv[r], -c00h * (float)h[r]);
            }
        }
        if ((lane & 63) == 0) reinterpret_cast<int *>(cr + BM * CRP2)[(rb - 1) * CRF + cb] = any ? 1 : 0;
    }
}

// Banded kernel matrices of the group's heads as MFMA A operands:
// tf[(a * c_q + i') * 64 + lane] = 8 fp16 of Theta_{i'} for row m = lane%16,
// columns k = 8*(lane/16) + s.
template <int CQ, int CK>
__device__ inline void build_theta_frags(f16x8 *tf, const float *th_s, int CH, int tid, int nt)
{
    constexpr int CKP = ((CK + 3) / 4) * 4;
    for (int i = tid; i < CH * CQ * 64; i += nt) {
        const int lane = i % 64, ip = (i / 64) % CQ, a = i / (64 * CQ);
        const int m = lane & 15, k0 = 8 * (lane >> 4);
        f16x8 h;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const int jj = m + CK - 1 - (k0 + s8);
            const float t = (jj >= 0 && jj < CK) ? th_s[(a * CQ + ip) * CKP + jj] : 0.f;
            h[s8] = (f16_t)f16_clamp(t);
        }
        tf[(a * CQ + ip) * 64 + lane] = h;
    }
}

// Kernel fragments of one head, resident in registers: th[i'].
template <int CQ>
struct ThetaFrags {
    f16x8 f[CQ];
};

template <int CQ>
__device__ inline void load_theta_frags(ThetaFrags<CQ> &t, const f16x8 *tf, int lane)
{
#pragma unroll
    for (int ip = 0; ip < CQ; ++ip) t.f[ip] = tf[ip * 64 + lane];
}

// Eq. 4's exact indicator on the matrix-core stencil: the B operand of a lane
// holds tile columns 32kh + 8*(lane/16) + s (+16 for the second block) of the
// rows above the lane's output query; entries whose key lies in that query's
// future are cleared.  w[t][q] masks 16-bit pair q of block t.
struct ColMask {
    uint32_t w[2][4];
};

// tl: last window column (relative to 32kh + 8*(lane/16)) whose key is not in
// the future of the lane's output query
__device__ inline ColMask col_mask(int tl)
{
    ColMask m;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 16 * t + 2 * q;
            m.w[t][q] = (c <= tl ? 0x0000ffffu : 0u) | (c + 1 <= tl ? 0xffff0000u : 0u);
        }
    return m;
}

__device__ inline f16x8 and_mask(f16x8 v, const uint32_t (&w)[4])
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u = __builtin_bit_cast(u32x4, v);
    u[0] &= w[0];
    u[1] &= w[1];
    u[2] &= w[2];
    u[3] &= w[3];
    return __builtin_bit_cast(f16x8, u);
}

// Two 16-key output blocks (keys 32kh + 16t + 4*(lane/16) + r, t = 0,1) of row
// 16rw + lane%16, kernel fragments th(ip).  out[4t + r].
// With `cr`, the accumulators start from the centre-tap corrections of the
// lane's row where the producing logit block wrote them (centre product
// exact; see store_block_x).  hl: tile column of key 0 of the key tile.
template <int CQ, bool MASK, typename TH>
__device__ inline void stencil_mfma_f(const f16_t *x, int ph, int rho, int kh, TH th, const ColMask &cm, int lane,
                                      float out[8], const f16_t *cr = nullptr, int hl = 0)
{
    const int g4 = lane >> 4;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    if (cr) {
        // flags of the logit blocks holding the wave's output keys (tile
        // columns 32kh + hl ..., hl = tile column of key 0 of the key tile)
        const int rb = (rho - HALO) >> 4;
        const int *fl = reinterpret_cast<const int *>(cr + BM * CRP2) + rb * CRF;
        const int c_lo = (32 * kh + hl) >> 4;
        unsigned bits = 0;
#pragma unroll
        for (int q = 0; q < 3; ++q) bits |= (fl[c_lo + q] ? 1u : 0u) << q;
        if (bits) {
            const f16_t *crow = cr + (rho - HALO) * CRP2 + 32 * kh + 4 * g4;
            const f16x4 c0 = *reinterpret_cast<const f16x4 *>(crow);
            const f16x4 c1 = *reinterpret_cast<const f16x4 *>(crow + 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k0 = ((32 * kh + 4 * g4 + r + hl) >> 4) - c_lo;
                a0[r] = ((bits >> k0) & 1u) ? (float)c0[r] : 0.f;
                a1[r] = ((bits >> (k0 + 1)) & 1u) ? (float)c1[r] : 0.f;
            }
        }
    }
#pragma unroll
    for (int ip = 0; ip < CQ; ++ip) {
        const int off = (rho - ip) * ph + 32 * kh + 8 * g4;
        f16x8 x0 = *reinterpret_cast<const f16x8 *>(x + off);
        f16x8 x1 = *reinterpret_cast<const f16x8 *>(x + off + 16);
        if (MASK) {
            x0 = and_mask(x0, cm.w[0]);
            x1 = and_mask(x1, cm.w[1]);
        }
        const f16x8 t = th(ip);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(t, x0, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(t, x1, a1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        out[r] = a0[r];
        out[4 + r] = a1[r];
    }
}

// kernel fragments in registers
template <int CQ, bool MASK>
__device__ inline void stencil_mfma_reg(const f16_t *x, int ph, int rho, int kh, const ThetaFrags<CQ> &tfr,
                                        const ColMask &cm, int lane, float out[8], const f16_t *cr = nullptr,
                                        int hl = 0)
{
    stencil_mfma_f<CQ, MASK>(x, ph, rho, kh, [&](int ip) { return tfr.f[ip]; }, cm, lane, out, cr, hl);
}

// kernel fragments read from LDS (tf of one head)
template <int CQ, bool MASK>
__device__ inline void stencil_mfma(const f16_t *x, int ph, int rho, int kh, const f16x8 *tf, const ColMask &cm,
                                    int lane, float out[8], const f16_t *cr = nullptr, int hl = 0)
{
    stencil_mfma_f<CQ, MASK>(x, ph, rho, kh, [&](int ip) { return tf[ip * 64 + lane]; }, cm, lane, out, cr, hl);
}

// ---------------------------------------------------------------------------
// Logit tile of one head from the Q and K tiles in LDS.  Wave (rw, kh):
// own-row block 1+rw for column blocks kh, kh+2, ...; the waves with kh == 1
// also take the HALO block's column blocks rw, rw+4, ... (only if c_q > 1).
template <int D, int MODE, bool HL, int NCB, bool EX>
__device__ inline void logit_tile_lds(float *sbuf, int ph, const bf16_t *qbuf, const bf16_t *kbuf,
                                      const Params &p, int i0, int j0, const float *st_m, const float *st_il,
                                      int rw, int kh, int lane, f16_t *cr = nullptr, float c00 = 0.f,
                                      float c00h = 0.f)
{
    const int l16 = lane & 15, dq = frag_base<D>(lane);
    f16_t *x16 = reinterpret_cast<f16_t *>(sbuf);
    QFrag<D> qf, kf;
    {
        const bf16_t *qr = qbuf + (16 * (1 + rw) + l16) * kpitch<D>() + dq;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) qf.x[t] = *reinterpret_cast<const bf16x8 *>(qr + 16 * t);
    }
#pragma unroll
    for (int cb = kh; cb < NCB; cb += 2) {
        const bf16_t *kr = kbuf + (16 * cb + l16) * kpitch<D>() + dq;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + 16 * t);
        const f32x4 acc = qk_mfma<D>(kf, qf);
        if (HL)
            store_block_x<MODE>(x16, ph, 1 + rw, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, EX, lane, cr, c00,
                                c00h);
        else
            store_block<MODE>(sbuf, p.pitch, 1 + rw, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, EX, lane);
    }
    if (kh == 1 && p.c_q > 1) {
        const bf16_t *qr = qbuf + l16 * kpitch<D>() + dq;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) qf.x[t] = *reinterpret_cast<const bf16x8 *>(qr + 16 * t);
#pragma unroll
        for (int cb = rw; cb < NCB; cb += 4) {
            const bf16_t *kr = kbuf + (16 * cb + l16) * kpitch<D>() + dq;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + 16 * t);
            const f32x4 acc = qk_mfma<D>(kf, qf);
            if (HL)
                store_block_x<MODE>(x16, ph, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, EX, lane);
            else
                store_block<MODE>(sbuf, p.pitch, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, st_m, st_il, EX, lane);
        }
    }
}

// Same tile with the wave's Q fragments already in registers (own-row block
// and, for the waves that take it, the halo block).
template <int D, int MODE, bool HL, int NCB, bool EX>
__device__ inline void logit_tile_regq(float *sbuf, int ph, const QFrag<D> &qown, const QFrag<D> &qhalo,
                                       const bf16_t *kbuf, const Params &p, int i0, int j0, int rw, int kh,
                                       int lane, f16_t *cr = nullptr, float c00 = 0.f, float c00h = 0.f)
{
    const int l16 = lane & 15, dq = frag_base<D>(lane);
    f16_t *x16 = reinterpret_cast<f16_t *>(sbuf);
    QFrag<D> kf;
#pragma unroll
    for (int cb = kh; cb < NCB; cb += 2) {
        const bf16_t *kr = kbuf + (16 * cb + l16) * kpitch<D>() + dq;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + 16 * t);
        const f32x4 acc = qk_mfma<D>(kf, qown);
        if (HL)
            store_block_x<MODE>(x16, ph, 1 + rw, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane, cr,
                                c00, c00h);
        else
            store_block<MODE>(sbuf, p.pitch, 1 + rw, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane);
    }
    if (kh == 1 && p.c_q > 1) {
#pragma unroll
        for (int cb = rw; cb < NCB; cb += 4) {
            const bf16_t *kr = kbuf + (16 * cb + l16) * kpitch<D>() + dq;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) kf.x[t] = *reinterpret_cast<const bf16x8 *>(kr + 16 * t);
            const f32x4 acc = qk_mfma<D>(kf, qhalo);
            if (HL)
                store_block_x<MODE>(x16, ph, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane);
            else
                store_block<MODE>(sbuf, p.pitch, 0, cb, acc, i0, j0, p.hl, p.T, p.sc, nullptr, nullptr, EX, lane);
        }
    }
}

template <int D>
__device__ inline void load_qfrags(QFrag<D> &qown, QFrag<D> &qhalo, const bf16_t *qbuf, int rw, int lane)
{
    const int l16 = lane & 15, dq = frag_base<D>(lane);
    const bf16_t *qo = qbuf + (16 * (1 + rw) + l16) * kpitch<D>() + dq;
    const bf16_t *qh = qbuf + l16 * kpitch<D>() + dq;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        qown.x[t] = *reinterpret_cast<const bf16x8 *>(qo + 16 * t);
        qhalo.x[t] = *reinterpret_cast<const bf16x8 *>(qh + 16 * t);
    }
}

// Key-query stencil, 8 consecutive outputs of one row (same sum as stencil16,
// window entries t > tlim taken as 0).
template <int CQ, int CK>
__device__ inline void stencil8(const float *buf, int pitch, int rho, int col0, const float *th, int tlim,
                                float out[8])
{
    constexpr int NWIN = 8 + CK - 1;
    constexpr int NW4 = (NWIN + 3) / 4;
    constexpr int CK4 = (CK + 3) / 4;
#pragma unroll
    for (int o = 0; o < 8; ++o) out[o] = 0.f;
#pragma unroll 1
    for (int ip = 0; ip < CQ; ++ip) {
        const f32x4 *row = reinterpret_cast<const f32x4 *>(buf + (rho - ip) * pitch + col0);
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
        if (tlim < NWIN - 1) {
#pragma unroll
            for (int t = 0; t < NWIN; ++t) win[t] = (t <= tlim) ? win[t] : 0.f;
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
        for (int jj = 0; jj < CK; ++jj)
#pragma unroll
            for (int o = 0; o < 8; ++o) out[o] = __builtin_fmaf(tw[jj], win[o + CK - 1 - jj], out[o]);
    }
}

// keys of the 8 values: key0 + ko[o]
__device__ inline void stats_update8(const float x[8], int key0, const int ko[8], int query, float &m, float &l)
{
    float tmax = NEG_INF;
#pragma unroll
    for (int o = 0; o < 8; ++o)
        if (key0 + ko[o] <= query) tmax = fmaxf(tmax, x[o]);
    const float mn = fmaxf(m, tmax);
    if (mn == NEG_INF) return;
    float s = (m == NEG_INF) ? 0.f : l * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
    for (int o = 0; o < 8; ++o)
        if (key0 + ko[o] <= query) s += __builtin_amdgcn_exp2f(x[o] - mn);
    m = mn;
    l = s;
}

// merge of two partial (m, l) pairs
__device__ inline void merge2(float &m, float &l, float m2, float l2)
{
    const float mx = fmaxf(m, m2);
    if (mx == NEG_INF) return;
    l = (m == NEG_INF ? 0.f : l * __builtin_amdgcn_exp2f(m - mx)) +
        (m2 == NEG_INF ? 0.f : l2 * __builtin_amdgcn_exp2f(m2 - mx));
    m = mx;
}

// merge over the four lanes of a row (lane, lane^16, lane^32, lane^48)
__device__ inline void merge_lanes(float &m, float &l)
{
    float m2 = __shfl_xor(m, 16), l2 = __shfl_xor(l, 16);
    merge2(m, l, m2, l2);
    m2 = __shfl_xor(m, 32);
    l2 = __shfl_xor(l, 32);
    merge2(m, l, m2, l2);
}

// ---------------------------------------------------------------------------
// MS: key-query stencil on the matrix cores (fp16, c_k <= 17) instead of
// the fp32 VALU stencil.  The lane's 8 values are then the keys
// 32kh + 16t + 4*(lane/16) + r (slot 4t + r) instead of 32kh + 8*(lane/16) + o.
// EXACT: the key-query convolution before the softmax with Eq. 4's exact
// indicator (unmasked logit tile, per-row column limit in the stencil).
template <int D, int CH, int CQ, int CK, bool KQ_POST, bool MS, bool EXACT>
__global__ void __launch_bounds__(NT, 1) mta_fwd_v2(Params p)
{
    static_assert(!(EXACT && KQ_POST), "the exact indicator applies before the softmax only");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rw = wave & 3, kh = wave >> 2;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = blockIdx.x;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;
    constexpr int CK4 = (CK + 3) / 4;
    constexpr int CKP = CK4 * 4;
    // 16-wide column blocks of the logit tile (the host passes the same value in p.ncb)
    constexpr int NCB0 = (BN + CK - 1 + 15) / 16;
    constexpr int NCB = (MS && NCB0 < 5) ? 5 : NCB0;
    const int ph = pitch_hl(NCB);

    const Layout lay = layout(D, CH, CQ, CK, NCB, p.pitch, MS, KQ_POST);
    float *sbuf = reinterpret_cast<float *>(smem + lay.s_off);
    const f16_t *x16 = reinterpret_cast<const f16_t *>(sbuf);
    bf16_t *kbuf = reinterpret_cast<bf16_t *>(smem + lay.k_off);
    bf16_t *qbuf = reinterpret_cast<bf16_t *>(smem + lay.q_off);
    bf16_t *vbuf = reinterpret_cast<bf16_t *>(smem + lay.v_off);
    bf16x8 *pbuf = reinterpret_cast<bf16x8 *>(smem + lay.p_off);
    float *st_m = reinterpret_cast<float *>(smem + lay.st_off);
    float *st_il = st_m + CH * EXT_R;
    float *xs = reinterpret_cast<float *>(smem + lay.xs_off);  // [kh][a][row][2]
    float *th_s = reinterpret_cast<float *>(smem + lay.th_off);
    float *w_s = reinterpret_cast<float *>(smem + lay.w_off);
    float *gnx = reinterpret_cast<float *>(smem + lay.gn_off);  // [kh][a][row]
    f16x8 *tf = reinterpret_cast<f16x8 *>(smem + lay.tf_off);
    // before the softmax with the matrix-core stencil: centre-tap corrections
    f16_t *cr = (MS && !KQ_POST) ? reinterpret_cast<f16_t *>(smem + lay.cr_off) : nullptr;

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
    if (MS) {
        __syncthreads();
        build_theta_frags<CQ, CK>(tf, th_s, CH, tid, NT);
    }

    const int io = 16 * rw + l16;        // output row within the query tile
    const int qabs = i0 + io;
    const int rho = HALO + io;
    const int col0 = 32 * kh + 8 * g4;   // VALU stencil: first of the lane's 8 key columns
    const int qhalo = i0 - HALO + l16;   // query of halo row l16 (waves with rw == 0)
    // key (within the key tile) of each of the lane's 8 stencil outputs
    int ko[8];
#pragma unroll
    for (int o = 0; o < 8; ++o) ko[o] = MS ? 32 * kh + 16 * (o >> 2) + 4 * g4 + (o & 3) : col0 + o;
    int kc[8];  // key tile columns for the raw-logit statistics (post-softmax convolution)
#pragma unroll
    for (int o = 0; o < 8; ++o) kc[o] = col0 + o;

    Pref<D> pf;
    load_q<D>(pf, Q, i0, T, tid);
    load_k<D>(pf, K, 0, p.hl, krows, T, tid);
    store_q<D>(pf, qbuf, tid);
    store_k<D>(pf, kbuf, krows, tid);

    // ------------------------------ pass 1 ---------------------------------
    // Head-major: all key tiles of head a, then head a+1, so that the head's Q
    // fragments and kernel fragments stay in registers.
    float m_c[CH], l_c[CH], m_h[CH], l_h[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        m_c[a] = NEG_INF; l_c[a] = 0.f; m_h[a] = NEG_INF; l_h[a] = 0.f;
    }
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        QFrag<D> qown, qhal;
        ThetaFrags<MS ? CQ : 1> tfr;
        for (int kt = 0; kt <= qt; ++kt) {
            const int j0 = kt * BN;
            __syncthreads();
            // next phase: (a, kt+1), or (a+1, 0), or pass 2's first phase (head 0,
            // tile 0); issued early so the loads overlap this whole phase
            const bool last = kt == qt;
            const int an = last ? (a + 1 < CH ? a + 1 : 0) : a;
            const int ktn = last ? 0 : kt + 1;
            load_k<D>(pf, K + an * hstride, ktn * BN, p.hl, krows, T, tid);
            if (CH > 1 && last) load_q<D>(pf, Q + an * hstride, i0, T, tid);
            // with the matrix-core stencil the head's Q and kernel fragments stay in
            // registers; the VALU-stencil variant has no registers to spare for them
            if (MS && kt == 0) {
                load_qfrags<D>(qown, qhal, qbuf, rw, lane);
                load_theta_frags<MS ? CQ : 1>(tfr, tf + a * CQ * 64, lane);
            }
            if (!KQ_POST && MS)
                logit_tile_regq<D, RAW, true, NCB, EXACT>(sbuf, ph, qown, qhal, kbuf, p, i0, j0, rw, kh, lane, cr,
                                                          th_s[a * CQ * CKP + CK / 2],
                                                          (float)(f16_t)f16_clamp(th_s[a * CQ * CKP + CK / 2]));
            else if (MS)
                logit_tile_regq<D, RAW, false, NCB, false>(sbuf, ph, qown, qhal, kbuf, p, i0, j0, rw, kh, lane);
            else
                logit_tile_lds<D, RAW, false, NCB, EXACT>(sbuf, ph, qbuf, kbuf, p, i0, j0, nullptr, nullptr, rw, kh,
                                                          lane);
            __syncthreads();
            if (!KQ_POST) {
                float c[8];
                // Eq. 4's indicator: window columns past tl hold keys in this row's future
                const int tl = EXACT ? qabs - (j0 - p.hl + col0) : (1 << 30);
                if (MS) {
                    // wave-uniform: can any of the wave's window columns pass its first row?
                    if (EXACT && j0 - p.hl + 32 * kh + 47 > i0 + 16 * rw)
                        stencil_mfma_reg<MS ? CQ : 1, true>(x16, ph, rho, kh, tfr, col_mask(tl), lane, c, cr, p.hl);
                    else
                        stencil_mfma_reg<MS ? CQ : 1, false>(x16, ph, rho, kh, tfr, ColMask{}, lane, c, cr, p.hl);
                } else {
                    stencil8<CQ, CK>(sbuf, p.pitch, rho, col0, th_s + a * CQ * CKP, tl, c);
                }
                stats_update8(c, j0, ko, qabs, m_c[a], l_c[a]);
            } else {
                float x[8];
#pragma unroll
                for (int o = 0; o < 8; ++o) x[o] = sbuf[rho * p.pitch + p.hl + col0 + o];
                stats_update8(x, j0, kc, qabs, m_c[a], l_c[a]);
                if (rw == 0) {
#pragma unroll
                    for (int o = 0; o < 8; ++o) x[o] = sbuf[l16 * p.pitch + p.hl + col0 + o];
                    stats_update8(x, j0, kc, qhalo, m_h[a], l_h[a]);
                }
            }
            store_k<D>(pf, kbuf, krows, tid);
            if (CH > 1 && last) store_q<D>(pf, qbuf, tid);
        }
    }

    // merge the statistics: lanes of a row, then the two key halves via LDS
    float M[CH], IL[CH];
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        merge_lanes(m_c[a], l_c[a]);
        if (KQ_POST) merge_lanes(m_h[a], l_h[a]);
    }
    if (g4 == 0) {
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            float *x = xs + ((kh * CH + a) * EXT_R) * 2;
            x[2 * rho] = m_c[a];
            x[2 * rho + 1] = l_c[a];
            if (KQ_POST && rw == 0) {
                x[2 * l16] = m_h[a];
                x[2 * l16 + 1] = l_h[a];
            }
        }
    }
    __syncthreads();
    if (!KQ_POST) {
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            const float *x0 = xs + ((0 * CH + a) * EXT_R) * 2;
            const float *x1 = xs + ((1 * CH + a) * EXT_R) * 2;
            float m = x0[2 * rho], l = x0[2 * rho + 1];
            merge2(m, l, x1[2 * rho], x1[2 * rho + 1]);
            M[a] = m;
            IL[a] = 1.0f / l;
        }
    } else {
        for (int i = tid; i < CH * EXT_R; i += NT) {
            const int a = i / EXT_R, r = i % EXT_R;
            const float *x0 = xs + ((0 * CH + a) * EXT_R) * 2;
            const float *x1 = xs + ((1 * CH + a) * EXT_R) * 2;
            float m = x0[2 * r], l = x0[2 * r + 1];
            merge2(m, l, x1[2 * r], x1[2 * r + 1]);
            // rows the convolution does not reach, or above the sequence start, stay zero
            const bool live = (r >= HALO - (CQ - 1)) && (i0 - HALO + r >= 0);
            st_m[i] = live ? m : 0.f;
            st_il[i] = live ? 1.0f / l : 0.f;
        }
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            M[a] = 0.f;
            IL[a] = 0.f;
        }
    }
    // (the first barrier of pass 2 publishes st_m / st_il)

    // ------------------------------ pass 2 ---------------------------------
    f32x4 acc[CH][D / 32];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) acc[a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int dbase = kh * (D / 2);

    // P.V of one head: the A operand (probabilities of 16 rows x 32 keys per
    // chunk) comes from the exchange buffer, B from the row-major V tile via
    // transposing loads, with the same key order as the producing lanes.
    auto pv = [&](int a, f32x4(&ac)[D / 32]) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 av = pbuf[((a * 4 + rw) * 2 + c) * 64 + lane];
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
                // keys of slots 0-3 and 4-7, matching the producing lanes' order
                const int kb0 = MS ? 32 * c + 4 * g4 : 32 * c + 8 * g4;
                const int kb1 = MS ? kb0 + 16 : kb0 + 4;
                const s16x4 u0 = lds_read_tr4(vbuf, vpitch<D>(), kb0, dbase + 16 * nb, l16);
                const s16x4 u1 = lds_read_tr4(vbuf, vpitch<D>(), kb1, dbase + 16 * nb, l16);
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 u = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                const bf16x8 bv = __builtin_bit_cast(bf16x8, u);
                ac[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, ac[nb], 0, 0, 0);
            }
        }
    };

    float pr[CH][8];
    for (int kt = 0; kt <= qt; ++kt) {
        const int j0 = kt * BN;
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            __syncthreads();
            // next phase (kt, a+1) or (kt+1, 0): its K, Q and the V tile its P.V
            // reads; issued early so the loads overlap this whole phase
            const int an = (a + 1 < CH) ? a + 1 : 0;
            const int ktn = (a + 1 < CH) ? kt : kt + 1;
            const bool more = ktn <= qt;
            if (more) {
                load_k<D>(pf, K + an * hstride, ktn * BN, p.hl, krows, T, tid);
                if (CH > 1) load_q<D>(pf, Q + an * hstride, i0, T, tid);
            }
            if (ktn >= 1) load_v<D>(pf, V + an * hstride, (ktn - 1) * BN, T, tid);
            if (KQ_POST)
                logit_tile_lds<D, PROB, MS, NCB, false>(sbuf, ph, qbuf, kbuf, p, i0, j0, st_m + a * EXT_R,
                                                        st_il + a * EXT_R, rw, kh, lane);
            else
                logit_tile_lds<D, RAW, MS, NCB, EXACT>(sbuf, ph, qbuf, kbuf, p, i0, j0, nullptr, nullptr, rw, kh,
                                                       lane, cr, th_s[a * CQ * CKP + CK / 2],
                                                       (float)(f16_t)f16_clamp(th_s[a * CQ * CKP + CK / 2]));
            if (kt > 0) pv(a, acc[a]);
            __syncthreads();

            float c[8];
            const int tl = EXACT ? qabs - (j0 - p.hl + col0) : (1 << 30);
            if (MS) {
                if (EXACT && j0 - p.hl + 32 * kh + 47 > i0 + 16 * rw)
                    stencil_mfma<CQ, true>(x16, ph, rho, kh, tf + a * CQ * 64, col_mask(tl), lane, c, cr, p.hl);
                else
                    stencil_mfma<CQ, false>(x16, ph, rho, kh, tf + a * CQ * 64, ColMask{}, lane, c, cr, p.hl);
            } else {
                stencil8<CQ, CK>(sbuf, p.pitch, rho, col0, th_s + a * CQ * CKP, tl, c);
            }
#pragma unroll
            for (int o = 0; o < 8; ++o) {
                const bool causal = j0 + ko[o] <= qabs;
                if (KQ_POST)
                    pr[a][o] = causal ? c[o] : 0.f;  // Mask_0 after the convolution
                else
                    pr[a][o] = causal ? __builtin_amdgcn_exp2f(c[o] - M[a]) * IL[a] : 0.f;
            }
            if (a == CH - 1) {
                // head mix after the softmax (Eq. 7), then publish for P.V
#pragma unroll
                for (int ao = 0; ao < CH; ++ao) {
                    bf16x8 v8;
#pragma unroll
                    for (int o = 0; o < 8; ++o) {
                        float s = 0.f;
#pragma unroll
                        for (int bb = 0; bb < CH; ++bb) s = __builtin_fmaf(w_s[ao * CH + bb], pr[bb][o], s);
                        v8[o] = (bf16_t)s;
                    }
                    pbuf[((ao * 4 + rw) * 2 + kh) * 64 + lane] = v8;
                }
            }
            if (more) {
                store_k<D>(pf, kbuf, krows, tid);
                if (CH > 1) store_q<D>(pf, qbuf, tid);
            }
            if (ktn >= 1) store_v<D>(pf, vbuf, tid);
        }
    }
    // P.V of the last key tile, one head at a time through the V buffer
#pragma unroll
    for (int a = 0; a < CH; ++a) {
        __syncthreads();
        pv(a, acc[a]);
        if (a + 1 < CH) {
            load_v<D>(pf, V + (a + 1) * hstride, qt * BN, T, tid);
            __syncthreads();
            store_v<D>(pf, vbuf, tid);
        }
    }

    // ---------------- epilogue: GroupNorm over d, depth scale, store -------
    // acc[a][nb][r] = O[row 16*rw + 4*g4 + r][col dbase + 16*nb + l16]
    float mu[CH][4];
#pragma unroll
    for (int a = 0; a < CH; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) s += acc[a][nb][r];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 8);
            if (l16 == 0) gnx[(kh * CH + a) * BM + 16 * rw + 4 * g4 + r] = s;
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
            float v2 = 0.f;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) {
                const float dl = acc[a][nb][r] - mu[a][r];
                v2 = __builtin_fmaf(dl, dl, v2);
            }
            v2 += __shfl_xor(v2, 1);
            v2 += __shfl_xor(v2, 2);
            v2 += __shfl_xor(v2, 4);
            v2 += __shfl_xor(v2, 8);
            if (l16 == 0) gnx[(kh * CH + a) * BM + 16 * rw + 4 * g4 + r] = v2;
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

template <int D, int CH, int CQ, int CK, bool POST, bool MS, bool EXACT>
hipError_t launch(const Params &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_v2<D, CH, CQ, CK, POST, MS, EXACT>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p);
    return hipGetLastError();
}

}  // namespace v2
}  // namespace mta
