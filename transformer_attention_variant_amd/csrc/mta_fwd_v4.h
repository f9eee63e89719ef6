// mta_fwd_v4.h — MTA forward with head-split waves, bf16, d = 128, for the
// kernel sizes instantiated in mta_inst_v4.hip (page "Multi-Token Attention —
// Paper Graph", section 3.4, "Key-Query Convolution", "Head Mixing
// Convolution" Eq. 7, "Group Normalization with Sigmoid Gating").  A
// workgroup owns two heads: a group of two (c_h = 2, head mix after the
// softmax), two single-head groups (NOMIX), one output pair of a group of
// 4, 8 or 16 heads (QUAD), or a group of two whose head mix precedes the softmax (C3D,
// as a 3D convolution).  One pass with the key-query convolution before the
// softmax (two-pass masks or Eq. 4's exact indicator), two passes with it
// after the softmax (POST); PREP is the gradient-preparation variant.
//
// A two-pass softmax walks the key tiles twice: once for each row's softmax
// statistics, once for the probabilities.  Before the softmax the statistics
// are kept online instead.  Post-softmax mixing combines NORMALISED maps of
// different heads, O^a = sum_b w_ab P^b V^a with P^b = exp(C^b - m_b) / l_b, and l_b is only
// known at the end, so the kernel keeps one accumulator per (source head b,
// output head a), U_{b,a} = sum_j exp(C^b_j - m_b) V^a_j (rescaled when m_b
// grows), and forms O^a = sum_b w_ab U_{b,a} / l_b in the epilogue: c_h^2
// accumulators and c_h times the P.V work instead of a whole first pass.  The
// work of a key tile is split by head:
//   wave (rw, s), rw = 0..3, s = 0..1, owns query rows 16rw.. of the tile.
//   In the logit product and the stencil it works on head s only, over all 64
//   keys of the tile, so the row maxima need no exchange between waves and
//   the head's banded kernel matrices stay in its registers.  In P.V it owns
//   the d-columns [64s, 64s + 64) of every (source b, output a) pair.
// Per key tile t there are two barriers, each publishing LDS writes only, and
// the P.V of a tile runs one phase late, beside the next tile's logit products:
//   A | K tiles of t, V tiles and probabilities of t - 1 are in LDS: rescale
//     | of the accumulators, P.V of t - 1; logit tiles of both heads -> LDS
//     | (fp16)
//   B | the K tiles of t + 1 and the V tiles of t start loading (DMA);
//     | stencil, Mask_-inf, row maximum, rescale factor, probabilities -> LDS
// The key-query convolution runs on the matrix cores with fp16 operands (the
// logit tile and the kernel taps rounded to nearest, 11 significant bits) and
// fp32 accumulation: one product per kernel row and output block.  Before the
// softmax the centre tap (the largest one of a kernel near the identity) is
// exact: the logit phase also writes the logits at the output positions to a
// centre-tap plane in LDS, and the stencil's accumulators start from the
// centre tap times those logits in fp32.
#pragma once

#include <type_traits>

#include "mta_tiles.h"

namespace mta {
namespace v4 {

constexpr int NT = 512;  // 8 waves, two per SIMD
using tile::swz_k;
using tile::swz_v;
using tile::barrier_lds;
using tile::vread_tr4;
using tile::lds_void_p;

constexpr int CH = 2;
constexpr int D = 128;
constexpr int NCB = 5;          // 16-key column blocks of the logit tile (80 columns)
constexpr int XP = 16 * NCB;    // fp16 pitch of the logit tiles (conflict-free stencil reads)
constexpr int KROWS = 16 * NCB; // K rows per head (key halo included)
// Tile column 0 is key j0 - XL (XL >= the convolution's left reach, c_k <= 17):
// the 16-key output blocks then sit at 16-byte-aligned tile columns 16t + XL,
// and the shared logit column block of consecutive key tiles still lines up.
constexpr int XL = 8;
// Centre-tap plane (before the softmax): row io of the query tile, output key o
// of the key tile at column o (o >= 8), keys 0..7 at columns 0..7 or 64..71 by
// key-tile parity (they are produced one key tile early).  The forward keeps
// the logits there in fp32; the gradient-preparation variant, short of LDS,
// keeps the fp16 rounding residuals and reads the rounded part from the
// logit tile.
constexpr int CRP = 72;

struct Layout {
    int x_off, k_off, v_off, qh_off, p_off, al_off, fl_off, gn_off, w_off, th_off, st_off, cr_off, total;
};

// prep: the gradient-preparation variant keeps P as bf16 high part and
// remainder (a second probability buffer)
__host__ __device__ inline Layout layout(int cq, int ck, bool prep = false, bool post = false, bool c3d = false)
{
    Layout L;
    int o = 0;
    L.x_off = o;  o += CH * EXT_R * XP * 2;       // logit tiles of both heads, fp16
    L.k_off = o;  o += CH * KROWS * D * 2;        // K tiles (swizzled rows)
    L.v_off = o;  o += CH * BN * D * 2;           // V tiles (swizzled rows)
    L.qh_off = o; o += CH * HALO * D * 2;         // Q rows above the query tile
    L.p_off = o;  o += (prep ? 2 : 1) * CH * 4 * 2 * 64 * 16;  // probabilities [plane][b][rw][k-step][lane] x 8 bf16
    L.al_off = o; o += CH * BM * 4;               // rescale factors [b][row]; at the end 1/l
    L.fl_off = o; o += CH * 4 * 4;                // [b][rw]: some factor of the 16 rows differs from 1
    L.gn_off = o; o += 2 * CH * BM * 4;           // GroupNorm partial sums [d half][a][row]
    L.w_off = o;  o += 16;                        // the group's 2x2 mixing matrix
    L.th_off = o; o += (((c3d ? CH : 1) * CH * cq * ((ck + 3) & ~3) + 3) & ~3) * 4;  // [a][(b)][row][col]
    // post: softmax statistics of the tile rows and the rows above them
    // (maximum, 1/sum: [h][row]) and the halo rows' partial statistics
    // ([h][key block][row][maximum, sum])
    L.st_off = o; o += post ? (2 * CH * EXT_R + CH * 4 * 16 * 2) * 4 : 0;
    // before the softmax: the centre-tap plane (fp32 logits; prep: fp16 residuals)
    L.cr_off = o; o += post ? 0 : CH * BM * CRP * (prep ? 2 : 4);
    L.total = o;
    return L;
}

// An offset the compiler must recompute where it is used: keeps it from holding
// the four lane addresses of every halo fragment load live across the loop.
__device__ inline int fresh(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// DMA of the same rows of a K or V tile for both heads of the group: piece i
// (1 KB = 4 rows) of head i / PER; wave w issues pieces w, w + 8, ... so that
// every wave issues the same number (its vmcnt bookkeeping is uniform).
template <bool VTILE, int NROWS>
__device__ inline void dma_pair(bf16_t *lds, const bf16_t *g, size_t hstride, int key0, int T, int wave, int lane)
{
    constexpr int PER = NROWS / 4;
    static_assert((CH * PER) % 8 == 0, "equal share per wave");
#pragma unroll
    for (int k = 0; k < CH * PER / 8; ++k) {
        const int i = wave + 8 * k, h = i / PER, piece = i % PER;
        const int row = 4 * piece + (lane >> 4), pc = lane & 15;
        const int c = pc ^ (VTILE ? swz_v(row) : swz_k(row));
        int key = key0 + row;
        key = key < 0 ? 0 : (key >= T ? T - 1 : key);
        // wave-uniform head base + 32-bit lane offset (scalar-base addressing)
        const char *gh = reinterpret_cast<const char *>(g + h * hstride);
        const unsigned off = (unsigned)key * (D * 2) + 16u * (unsigned)c;
        __builtin_amdgcn_global_load_lds((const void *)(gh + off), (lds_void_p)(lds + h * NROWS * D + 512 * piece),
                                         16, 0, 0);
    }
}
// all of this wave's global loads (its DMA pieces included) have landed
__device__ inline void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

typedef _Float16 f16_t;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// fp16 operand of the stencil: magnitudes past the fp16 range are clamped to
// its largest finite value (never inf, so a zero tap never meets an infinity)
__device__ inline float f16_range(float x) { return __builtin_amdgcn_fmed3f(x, -65504.f, 65504.f); }

// fp16 P.V: a wave's own pieces of a V tile (those dma_pair<true, NROWS>
// gave it: 1 KB each, lane l's 16 bytes at 16 l), bf16 -> fp16 in place,
// elementwise, so the rows' swizzle is kept.  Exact for 2^-14 <= |v| <= 65504
// (bf16's 8 significant bits fit fp16's 11); smaller magnitudes round to the
// fp16 subnormal grid (absolute error <= 2^-25), larger ones clamp to 65504.
template <int NROWS>
__device__ inline void v_to_f16(bf16_t *lds, int wave, int lane)
{
    constexpr int PER = NROWS / 4;
#pragma unroll 1
    for (int k = 0; k < CH * PER / 8; ++k) {  // one piece at a time: few registers
        const int i = wave + 8 * k, h = i / PER, piece = i % PER;
        bf16x8 *cell = reinterpret_cast<bf16x8 *>(lds + h * NROWS * D + 512 * piece) + lane;
        const bf16x8 x = *cell;
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (f16_t)f16_range((float)x[e]);
        *cell = __builtin_bit_cast(bf16x8, y);
    }
}

// fp16 logit tiles: row rho (0..EXT_R-1) holds 80 columns in ten 16-byte
// chunks; chunk c of row rho is stored at chunk c ^ ((rho >> 2) & 1).  With the
// 160-byte row pitch this keeps the stencil's 16-byte reads and the paired
// 16-byte block stores below free of bank conflicts (ds_write_b128 serves 8
// consecutive lanes per pass over a 128-byte bank window).
// With c_q = 8 the kernel keeps the unswizzled layout and stores each block by
// itself (8 bytes per lane): the pair exchange needs registers that kernel
// does not have to spare.
template <int CQ>
__device__ inline int xchunk(int rho, int c) { return CQ < 8 ? c ^ ((rho >> 2) & 1) : c; }

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A 16x16 block of raw logits Q K^T (lane: tile row rb*16 + lane%16, columns
// cb*16 + 4*(lane/16) + r) converted to fp16 with Mask_0 and the zero padding
// outside [0, T) applied (with `exact` only the padding); MASKED = false when
// the caller knows that every entry of the block is kept.  The convolution
// being linear, the factor log2(e)/sqrt(d) is applied to the kernel taps.
// `xs` receives the masked logits in fp32 (for the centre-tap plane).
template <bool MASKED>
__device__ inline u32x2 cvt_block(int rb, int cb, f32x4 acc, int i0, int j0, int hl, int T, bool exact, int lane,
                                  f32x4 &xs)
{
    const int rho = rb * 16 + (lane & 15);
    const int e0 = cb * 16 + 4 * (lane >> 4);
    const int qi = i0 - HALO + rho;
    const int kmax = exact ? T - 1 : qi;
    // block-uniform: every entry kept and inside [0, T), or not
    const int q_lo = i0 - HALO + rb * 16, k_lo = j0 - hl + cb * 16;
    const bool all_ok = (k_lo >= 0) && (k_lo + 15 <= (exact ? T - 1 : q_lo)) && (q_lo >= 0) && (q_lo + 15 < T);
    float xv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = acc[r];
        if (MASKED && !all_ok) {
            const int kj = j0 - hl + e0 + r;
            const bool ok = (kj >= 0) && (kj <= kmax) && (qi >= 0) && (qi < T);
            v = ok ? v : 0.f;
        }
        xs[r] = v;
        xv[r] = f16_range(v);
    }
    const f16x4 h = {(f16_t)xv[0], (f16_t)xv[1], (f16_t)xv[2], (f16_t)xv[3]};
    return __builtin_bit_cast(u32x2, h);
}

// Centre-tap plane write of an own-row logit block (tile columns 16cb +
// 4(lane/16) + r hold output keys 16cb + 4(lane/16) - XL + r): keys 0..7 go to
// the region of this tile's parity, keys 64..71 (the next tile's 0..7) to the
// other parity's region, and keys -8..-1 (only in the first tile, whose block 0
// is computed; nobody reads them) to the other region too, before block 4's
// writes land there in the same wave's program order.  The column is plain
// arithmetic on the lane half (no per-lane masks to keep live).  F32: the
// logits xs; else the fp16 residuals of their rounding h.
template <int CB, bool F32>
__device__ inline void store_centre(void *crow, f32x4 xs, u32x2 h, int t, int lane)
{
    const int g4 = lane >> 4, hi = g4 >> 1, q = 4 * (g4 & 1);
    const int cur = (t & 1) ? 64 : 0, other = 64 - cur;
    int col;
    if constexpr (CB == 0)
        col = q + other + hi * (cur - other);
    else if constexpr (CB == NCB - 1)
        col = q + 56 + hi * (other - 56);
    else
        col = 16 * CB + 4 * g4 - XL;
    if constexpr (F32) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(crow) + col) = xs;
    } else {
        const f16x4 hh = __builtin_bit_cast(f16x4, h);
        const f16x4 e = {(f16_t)(f16_range(xs[0]) - (float)hh[0]), (f16_t)(f16_range(xs[1]) - (float)hh[1]),
                         (f16_t)(f16_range(xs[2]) - (float)hh[2]), (f16_t)(f16_range(xs[3]) - (float)hh[3])};
        *reinterpret_cast<u32x2 *>(reinterpret_cast<f16_t *>(crow) + col) = __builtin_bit_cast(u32x2, e);
    }
}

// The same block as probabilities of the softmax before a post-softmax
// convolution: exp2(sc * S - m) * il with the row's statistics (m: maximum of
// sc * S over its causal keys, il: 1 / sum), 0 for keys in the row's future and
// outside [0, T) (entries whose exp2 may be out of range are selected away,
// never multiplied).
template <bool MASKED>
__device__ inline u32x2 cvt_prob(int rb, int cb, f32x4 acc, int i0, int j0, int hl, int T, float m, float il,
                                 float sc, int lane)
{
    const int rho = rb * 16 + (lane & 15);
    const int e0 = cb * 16 + 4 * (lane >> 4);
    const int qi = i0 - HALO + rho;
    const int q_lo = i0 - HALO + rb * 16, k_lo = j0 - hl + cb * 16;
    const bool all_ok = (k_lo >= 0) && (k_lo + 15 <= q_lo) && (q_lo >= 0) && (q_lo + 15 < T);
    float xv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], sc, -m)) * il;
        if (MASKED && !all_ok) {
            const int kj = j0 - hl + e0 + r;
            const bool ok = (kj >= 0) && (kj <= qi) && (qi >= 0) && (qi < T);
            v = ok ? v : 0.f;
        }
        xv[r] = v;
    }
    const f16x4 h = {(f16_t)xv[0], (f16_t)xv[1], (f16_t)xv[2], (f16_t)xv[3]};
    return __builtin_bit_cast(u32x2, h);
}

// Store two converted blocks X and Y (tile bases xX, xY; row blocks, column
// blocks): lane groups 2k and 2k+1 hold keys 8k..8k+3 and 8k+4..8k+7 of the same
// row; one exchange between them (v_permlane16_swap) leaves the even group with
// 8 keys of X and the odd group with 8 keys of Y, and every lane stores 16
// bytes.  With `one`, Y is absent and the odd groups store nothing.
template <int CQ>
__device__ inline void store_pair(f16_t *xX, int rbX, int cbX, u32x2 vX, f16_t *xY, int rbY, int cbY, u32x2 vY,
                                  int lane, bool one = false)
{
    if (CQ >= 8) {
        // unpaired: each block by itself, 8 bytes per lane
        const int l16 = lane & 15, g4 = lane >> 4;
        *reinterpret_cast<u32x2 *>(xX + (rbX * 16 + l16) * XP + 16 * cbX + 4 * g4) = vX;
        if (!one) *reinterpret_cast<u32x2 *>(xY + (rbY * 16 + l16) * XP + 16 * cbY + 4 * g4) = vY;
        return;
    }
    const auto s0 = __builtin_amdgcn_permlane16_swap(vX[0], vY[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(vX[1], vY[1], false, false);
    const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
    const int g4 = lane >> 4;
    const bool odd = g4 & 1;
    const int rho = (odd ? rbY : rbX) * 16 + (lane & 15);
    f16_t *x = odd ? xY : xX;
    const int c = 2 * (odd ? cbY : cbX) + (g4 >> 1);
    if (!(one && odd)) *reinterpret_cast<u32x4 *>(x + rho * XP + 8 * xchunk<CQ>(rho, c)) = w;
}

__device__ inline f16x8 and_mask16(f16x8 v, const uint32_t (&w)[4])
{
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] &= w[q];
    return __builtin_bit_cast(f16x8, u);
}

// maximum / sum over the four lanes l16 + 16 g4 holding one row
__device__ inline float row_max4(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float row_sum4(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Eq. 4's indicator for one 16-key output block: the B operand of a lane holds
// window columns 8*(lane/16) + s of the rows above its output query; entries
// whose key is in that query's future (window column > tl) are cleared.
__device__ inline void block_mask(int tl, uint32_t (&w)[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w[q] = (2 * q <= tl ? 0x0000ffffu : 0u) | (2 * q + 1 <= tl ? 0xffff0000u : 0u);
}

// Q K^T of a 16x16 block over d = 128 (one accumulation chain).
__device__ inline f32x4 qk(const QFrag<D> &kf, const QFrag<D> &qf)
{
    f32x4 a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.x[0], qf.x[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int t = 1; t < D / 32; ++t) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf.x[t], qf.x[t], a, 0, 0, 0);
    return a;
}

// Accumulator start of the stencil's output block t for the lane (keys
// 16t + 4*(lane/16) + r of its row): the centre tap (query offset 0, key
// offset 0) times the logit itself, in fp32; the banded matrices leave that tap
// out.  CORR = 1: the logits from the fp32 plane; CORR = 2: the fp16 logit
// tile's value plus its fp16 residual.  par: the column of keys 0..7 of this
// key tile (0 or 64).
template <int CQ, int CORR>
__device__ inline f32x4 centre_init(const f16_t *x, int rho, const void *crow, int t, int par, float c00, int lane)
{
    const int g4 = lane >> 4, o = 16 * t + 4 * g4;
    // keys 0..7 (block 0, lanes 0..31) sit at the tile parity's column
    const int col = t == 0 ? o + (1 - (g4 >> 1)) * par : o;
    if constexpr (CORR == 1) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(crow) + col);
        return f32x4{c00 * v[0], c00 * v[1], c00 * v[2], c00 * v[3]};
    } else {
        const f16x4 e = __builtin_bit_cast(f16x4, *reinterpret_cast<const u32x2 *>(
                                                      reinterpret_cast<const f16_t *>(crow) + col));
        // tile column o + XL: 16-byte chunk (o + XL) / 8, half (o + XL) % 8 = 4 (g4 & 1)
        const f16x4 h = *reinterpret_cast<const f16x4 *>(x + rho * XP + 8 * xchunk<CQ>(rho, (o + XL) >> 3) +
                                                         4 * (g4 & 1));
        f32x4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = c00 * ((float)h[k] + (float)e[k]);
        return r;
    }
}

// Key-query stencil of the 16 rows of this wave (tile row rho = HALO + 16rw +
// lane%16) over all 64 keys of the tile: output block t covers keys 16t..16t+15
// and reads the 32-column window starting at tile column 16t (keys j0 - XL +
// 16t ...).  One fp16 product per kernel row on the matrix cores.  out[4t + r]
// is key 16t + 4*(lane/16) + r.  With CORR the accumulators start from the
// centre tap's term (centre_init).  With MASK, Eq. 4's indicator: tl0
// is the last window column of block 0 (relative to 8*(lane/16)) whose key is
// not in the future of the lane's output query; the blocks are then taken two
// at a time with their masks built just before use.
template <int CQ, bool MASK, int CORR>
__device__ inline void stencil64(const f16_t *x, int rho, const f16x8 (&tf)[CQ], int tl0, const void *crow,
                                 int par, float c00, int lane, float out[16])
{
    const int g4 = lane >> 4;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = CORR ? centre_init<CQ, CORR>(x, rho, crow, t, par, c00, lane) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (MASK) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t mk[4];
            block_mask(tl0 - 16 * t, mk);
#pragma unroll
            for (int ip = 0; ip < CQ; ++ip) {
                const int r = rho - ip;
                const f16x8 xv = *reinterpret_cast<const f16x8 *>(x + r * XP + 8 * xchunk<CQ>(r, g4) + 16 * t);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tf[ip], and_mask16(xv, mk), acc[t], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int ip = 0; ip < CQ; ++ip)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = rho - ip;
                const f16x8 xv = *reinterpret_cast<const f16x8 *>(x + r * XP + 8 * xchunk<CQ>(r, g4) + 16 * t);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tf[ip], xv, acc[t], 0, 0, 0);
            }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[4 * t + r] = acc[t][r];
}

// The 3D form's stencil (two-pass masks): both heads' logit tiles x and x2,
// each through its own banded kernel matrices, accumulated into one output
// that starts from the own head's (x) centre-tap term (fp32 plane).
template <int CQ>
__device__ inline void stencil64_pair(const f16_t *x, const f16_t *x2, int rho, const f16x8 (&tf)[CQ],
                                      const f16x8 (&tf2)[CQ], const void *crow, int par, float c00, int lane,
                                      float out[16])
{
    const int g4 = lane >> 4;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = centre_init<CQ, 1>(x, rho, crow, t, par, c00, lane);
#pragma unroll
    for (int ip = 0; ip < CQ; ++ip)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = rho - ip, off = r * XP + 8 * xchunk<CQ>(r, g4) + 16 * t;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tf[ip], *reinterpret_cast<const f16x8 *>(x + off), acc[t],
                                                            0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tf2[ip], *reinterpret_cast<const f16x8 *>(x2 + off),
                                                            acc[t], 0, 0, 0);
        }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[4 * t + r] = acc[t][r];
}

// Extra pointers of the gradient-preparation variant (PREP): dY, the
// workspace of the backward (row statistics, D, dO as bf16 high part and
// remainder) and the GroupNorm / gate gradients it accumulates into.
struct PrepArgs {
    const bf16_t *dout;
    float *ws_m, *ws_il, *ws_D;
    bf16_t *ws_dO, *ws_dOl;
    float *dgn_w, *dgn_b, *dgate;
};

// PREP: instead of the output, the epilogue writes what the backward's main
// kernel needs (the same quantities as bwd::mta_bwd_prep: per-row statistics,
// the GroupNorm backward dO, D^b = sum_a w_ab dO^a . (P^b V^a)) and adds the
// GroupNorm and gate gradients.
// POST: the key-query convolution after the softmax (then Mask_0), in two
// passes over the key tiles: the softmax statistics of the tile's rows and of
// the 16 rows above it first, then the probabilities of the extended tile ->
// fp16 stencil -> Mask_0 -> P.V; the head mix stays in the epilogue.
// C3D: the both-pre-softmax 3D convolution (kernel theta[g][a][b][i'][j'], p.theta)
// in place of the per-head one, with no head mix after the softmax: output head
// a's stencil sums over the logit tiles of both heads b, and only the P.V
// products of head a's probabilities with V^a are formed.  With p.head_pre the
// kernel is built from the per-head kernels and the pre-softmax head mix.
// NOMIX: head groups of one head (c_h = 1), taken two at a time: the two
// heads of the workgroup are neighbouring single-head groups, so only the
// U[a][a] products are formed and each output head is its own head's mixed map
// (the 1x1 mixing weight w_h, p.wmix[h]).  p.G and p.units count head pairs.
template <int CQ, int CK, bool EXACT, bool PREP = false, bool POST = false, bool C3D = false, bool NOMIX = false,
          bool QUAD = false, bool F16PV = false>
__global__ void __launch_bounds__(NT, 1) mta_fwd_v4(Params p, PrepArgs pa)
{
    static_assert(CK <= 17, "matrix-core stencil: 32-column window");
    static_assert(!(POST && (EXACT || PREP)), "post-softmax form: two-pass masks, forward only");
    static_assert(!(C3D && (EXACT || PREP || POST)), "3D form: two-pass masks, forward only");
    static_assert(!(NOMIX && (C3D || PREP)), "single-head groups: the forward of the per-head kernels");
    static_assert(!(QUAD && (C3D || PREP || NOMIX)), "groups of four or more heads: the forward with the mix after the softmax");
    constexpr bool DIAG = C3D || NOMIX;  // output head a uses only source head a
    // PREP: probabilities kept to ~16 bits in P.V (a bf16 high part and the
    // bf16 remainder, two planes), as the gradients need.  F16PV: P.V in fp16
    // (11 significant bits against bf16's 8; V converted in LDS), for large
    // head groups, whose head mix would otherwise add up one bf16 rounding of
    // every source head's map, weighted by |w_ab|, however much the weighted
    // maps cancel
    static_assert(!(F16PV && PREP), "fp16 P.V: the forward");
    constexpr bool PP = PREP;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int pi = 0;  // QUAD: source pair of this sweep (see below)
    // QUAD: the finished sweeps' sum of this lane's output elements, kept in
    // its private memory between sweeps (volatile: memory, not registers)
    volatile float keep[QUAD ? CH * 4 * 4 : 1];
sweep:
    // QUAD: the thread and workgroup indices pass through an empty asm that
    // depends on the sweep, so that everything derived from them is computed
    // again in each sweep rather than held across both
    int tid0 = threadIdx.x, blk0 = blockIdx.x;
    if constexpr (QUAD) {
        asm volatile("" : "+v"(tid0) : "s"(pi));
        asm volatile("" : "+s"(blk0) : "s"(pi));
    }
    const int tid = tid0, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers and branches
    const int rw = wave & 3, hs = wave >> 2;  // row block; head (stencil) = d half (P.V)
    const int l16 = lane & 15, g4 = lane >> 4;
    const int L = blk0;
    const int unit = L % p.units;
    const int qt = p.n_qt - 1 - L / p.units;
    const int b = unit / p.G, g = unit % p.G;
    const int i0 = qt * BM;
    const int T = p.T;
    constexpr int CKP = ((CK + 3) / 4) * 4;

    const Layout lay = layout(CQ, CK, PP, POST, C3D);
    f16_t *xbuf = reinterpret_cast<f16_t *>(smem + lay.x_off);
    bf16_t *kbuf = reinterpret_cast<bf16_t *>(smem + lay.k_off);
    bf16_t *vbuf = reinterpret_cast<bf16_t *>(smem + lay.v_off);
    bf16_t *qhbuf = reinterpret_cast<bf16_t *>(smem + lay.qh_off);
    bf16x8 *pbuf = reinterpret_cast<bf16x8 *>(smem + lay.p_off);
    float *al = reinterpret_cast<float *>(smem + lay.al_off);   // [b][row]
    int *fl = reinterpret_cast<int *>(smem + lay.fl_off);       // [b][rw]
    float *gnx = reinterpret_cast<float *>(smem + lay.gn_off);  // [half][a][row]
    float *w_s = reinterpret_cast<float *>(smem + lay.w_off);
    float *th_s = reinterpret_cast<float *>(smem + lay.th_off);
    float *stm = reinterpret_cast<float *>(smem + lay.st_off);  // POST: [h][row] maximum (log2 domain)
    float *stil = stm + CH * EXT_R;                             // POST: [h][row] 1 / sum
    // before the softmax: the centre-tap plane [h][row][CRP] (fp32; PP: fp16 residuals)
    unsigned char *crbuf = smem + lay.cr_off;
    constexpr int CORR = POST ? 0 : (PP ? 2 : 1);

    // QUAD (groups of c_h = 2 * p.npair >= 4 heads): the workgroup owns output
    // heads h0, h0 + 1 (output pair g % npair of the group g / npair); O^a sums
    // over the group's source pairs, sum_s w_as U_{s,a} / l_s, one sweep over
    // the key tiles per source pair with the two-head machinery below (that
    // pair's logits, stencils and softmax statistics; P.V with the output
    // pair's V).  The running sum of the finished sweeps waits in each lane's
    // private memory (float32) until the last sweep adds it.
    const size_t hstride = (size_t)T * D;
    const int h0 = g * CH;
    const size_t base0 = ((size_t)b * p.H + h0) * hstride;
    const int grp = QUAD ? g / p.npair : g;
    const int hsrc0 = QUAD ? 2 * p.npair * grp + 2 * pi : h0;  // source heads of this sweep
    const size_t sbase = ((size_t)b * p.H + hsrc0) * hstride;
    const bf16_t *Q = reinterpret_cast<const bf16_t *>(p.q) + sbase;
    const bf16_t *K = reinterpret_cast<const bf16_t *>(p.k) + sbase;
    const bf16_t *V = reinterpret_cast<const bf16_t *>(p.v) + base0;

    // K of key tile 0 (POST: the statistics pass's 64 keys) and the Q rows above
    // the query tile, both heads; this wave's Q rows of its head in registers;
    // kernels and mixing matrix
    if constexpr (POST)
        dma_pair<false, BN>(kbuf, K, hstride, 0, T, wave, lane);
    else
        dma_pair<false, KROWS>(kbuf, K, hstride, -XL, T, wave, lane);
    dma_pair<false, HALO>(qhbuf, Q, hstride, i0 - HALO, T, wave, lane);
    // this wave's Q rows of its head (rows past the end: masked in the logit tile)
    const bf16_t *qrow = Q + hs * hstride + (size_t)((i0 + 16 * rw + l16) < T ? i0 + 16 * rw + l16 : T - 1) * D + 32 * g4;
    QFrag<D> qown;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) qown.x[t] = *reinterpret_cast<const bf16x8 *>(qrow + 8 * t);
    if constexpr (C3D) {
        // p.head_pre: the per-head kernels followed by the head mix before the
        // softmax, which by linearity is the 3D kernel w[g][a][b] * theta[h0 + b]
        for (int i = tid; i < CH * CH * CQ * CKP; i += NT) {
            const int ab = i / (CQ * CKP), r = (i / CKP) % CQ, c = i % CKP;
            float v = 0.f;
            if (c < CK)
                v = p.head_pre ? p.wmix[(size_t)g * CH * CH + ab] *
                                     p.theta[((size_t)(h0 + ab % CH) * CQ + r) * CK + c]
                               : p.theta[(((size_t)g * CH * CH + ab) * CQ + r) * CK + c];
            th_s[i] = v;
        }
        if (tid < CH * CH) w_s[tid] = (tid / CH == tid % CH) ? 1.f : 0.f;  // no mix after the softmax
    } else {
        for (int i = tid; i < CH * CQ * CKP; i += NT) {
            const int a = i / (CQ * CKP), r = (i / CKP) % CQ, c = i % CKP;
            th_s[i] = c < CK ? p.theta[((size_t)(hsrc0 + a) * CQ + r) * CK + c] : 0.f;
        }
        // w_s[a][s]: output head a of the pair, source head s of this sweep
        if (tid < CH * CH)
            w_s[tid] = NOMIX ? ((tid / CH == tid % CH) ? p.wmix[h0 + tid / CH] : 0.f)
                     : QUAD  ? p.wmix[((size_t)grp * 2 * p.npair + (h0 - 2 * p.npair * grp) + tid / CH) * 2 * p.npair +
                                      2 * pi + tid % CH]
                             : p.wmix[(size_t)g * CH * CH + tid];
    }
    wait_vm_all();
    __syncthreads();

    // Before the softmax the centre tap (i' = 0, j' = 0) of head hs's own
    // kernel is applied in fp32 to the logit itself (centre_init); the banded
    // matrices leave it out.  After the softmax the taps act on probabilities,
    // unscaled.
    const float c00 =
        POST ? 0.f : th_s[(C3D ? (hs * CH + hs) : hs) * CQ * CKP + CK / 2] * p.sc;
    const float kap = POST ? 1.f : p.sc;

    // banded kernel matrices of head hs (MFMA A operands, fp16):
    // row m = lane%16 (output key j0 + 16t + m), columns k = 8*(lane/16) + s of
    // the window (key j0 - XL + 16t + k), so j' = m + XL - k
    // (C3D: tf from source head hs, tfo from the other head, both into head hs;
    // the own centre tap is left out before the softmax)
    f16x8 tf[CQ], tfo[C3D ? CQ : 1];
#pragma unroll
    for (int ip = 0; ip < CQ; ++ip)
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const int jj = l16 + XL - (8 * g4 + s8) + CK / 2;
            const bool in = jj >= 0 && jj < CK && (POST || ip != 0 || jj != CK / 2);
            if constexpr (C3D) {
                const float t = in ? th_s[((hs * CH + hs) * CQ + ip) * CKP + jj] : 0.f;
                const bool in2 = jj >= 0 && jj < CK;  // the other head's centre tap stays
                const float u = in2 ? th_s[((hs * CH + (1 - hs)) * CQ + ip) * CKP + jj] : 0.f;
                tf[ip][s8] = (f16_t)f16_range(t * kap);
                tfo[ip][s8] = (f16_t)f16_range(u * kap);
            } else {
                const float t = in ? th_s[(hs * CQ + ip) * CKP + jj] : 0.f;
                tf[ip][s8] = (f16_t)f16_range(t * kap);
            }
        }

    const int io = 16 * rw + l16;  // the lane's stencil row within the query tile
    // its row of the centre-tap plane (before the softmax)
    void *crow = crbuf + (size_t)(hs * BM + io) * CRP * (PP ? 2 : 4);
    const int qabs = i0 + io;
    const int rho = HALO + io;
    const int dbase = 64 * hs;
    f16_t *xo = xbuf + hs * EXT_R * XP;
    int koff[4];  // swizzled chunk offsets of the K / Q-halo fragment reads
#pragma unroll
    for (int t = 0; t < 4; ++t) koff[t] = 8 * ((4 * g4 + t) ^ swz_k(l16));

    // POST, pass 1: running maximum and sum of sc * S over the causal keys, per
    // lane (its 16 keys of a tile) for row io of head hs and for halo row l16 of
    // head wave / 4 (key block wave % 4 of every tile); merged over the lanes
    // and the four halo waves at the end.  K tiles of 64 keys, double-buffered
    // in the K and V buffers (free in this pass).
    float pm_o = 0.f, pil_o = 0.f, pm_h = 0.f, pil_h = 0.f;
    if constexpr (POST) {
        const int hh = wave >> 2, hcb = wave & 3;
        constexpr float FLOOR = -1e30f;  // finite: a lane with no causal key yet keeps l = 0
        float m1 = FLOOR, l1 = 0.f, m2 = FLOOR, l2 = 0.f;
        auto update = [](float &m, float &l, const float *v, int n) {
            float mx = m;
            for (int o = 0; o < n; ++o) mx = fmaxf(mx, v[o]);
            float sum = 0.f;
            for (int o = 0; o < n; ++o) sum += __builtin_amdgcn_exp2f(v[o] - mx);  // exp2(-inf) = 0
            l = __builtin_fmaf(l, __builtin_amdgcn_exp2f(m - mx), sum);
            m = mx;
        };
        auto kload = [&](QFrag<D> &f, const bf16_t *rows, int cb) {
#pragma unroll
            for (int t = 0; t < 4; ++t) f.x[t] = *reinterpret_cast<const bf16x8 *>(rows + 16 * cb * D + koff[t]);
        };
        QFrag<D> hq;
        kload(hq, qhbuf + (hh * HALO + l16) * D, 0);
        const int qh = i0 - HALO + l16;  // the lane's halo row
        for (int t = 0; t <= qt; ++t) {
            const int j0 = t * BN;
            bf16_t *kb = (t & 1) ? vbuf : kbuf;
            wait_vm_all();
            __syncthreads();  // K(t) in LDS; every wave is done with the other buffer
            if (t < qt) dma_pair<false, BN>((t & 1) ? kbuf : vbuf, K, hstride, j0 + BN, T, wave, lane);
            float v[16];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                QFrag<D> kf;
                kload(kf, kb + (hs * BN + l16) * D, cb);
                const f32x4 acc = qk(kf, qown);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[4 * cb + r] = (j0 + 16 * cb + 4 * g4 + r <= qabs) ? acc[r] * p.sc : NEG_INF;
            }
            update(m1, l1, v, 16);
            {
                QFrag<D> kf;
                kload(kf, kb + (hh * BN + l16) * D, hcb);
                const f32x4 acc = qk(kf, hq);
                float w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = (j0 + 16 * hcb + 4 * g4 + r <= qh) ? acc[r] * p.sc : NEG_INF;
                update(m2, l2, w, 4);
            }
        }
        // merge the four lanes of each row (keys 4 * (lane / 16) + ...)
        const float mo = row_max4(m1), lo = row_sum4(l1 * __builtin_amdgcn_exp2f(m1 - mo));
        const float mh = row_max4(m2), lh = row_sum4(l2 * __builtin_amdgcn_exp2f(m2 - mh));
        float *hpart = stil + CH * EXT_R;  // [h][key block][row][maximum, sum]
        if (g4 == 0) {
            stm[hs * EXT_R + rho] = mo;
            stil[hs * EXT_R + rho] = lo > 0.f ? 1.0f / lo : 0.f;
            hpart[((hh * 4 + hcb) * 16 + l16) * 2 + 0] = mh;
            hpart[((hh * 4 + hcb) * 16 + l16) * 2 + 1] = lh;
        }
        __syncthreads();  // pass-1 reads of the K buffers and the partial statistics are done
        dma_pair<false, KROWS>(kbuf, K, hstride, -XL, T, wave, lane);  // pass 2's first K tiles
        if (tid < CH * 16) {
            // halo rows: the four key blocks of each
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
        pm_o = stm[hs * EXT_R + rho];
        pil_o = stil[hs * EXT_R + rho];
        pm_h = stm[hh * EXT_R + l16];
        pil_h = stil[hh * EXT_R + l16];
    }

    // U[b][a][nb][r]: rows 16rw + 4g4 + r, d-columns dbase + 16nb + l16
    f32x4 U[CH][CH][4];
#pragma unroll
    for (int s = 0; s < CH; ++s)
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) U[s][a][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = NEG_INF, l_run = 0.f;  // head hs, row io (l_run: this lane's 16 keys)

    // Two phases per key tile t (one more step drains the last P.V):
    //   A(t) | K(t), V(t-1), P(t-1) in LDS | logit tiles of t; rescale and P.V of t-1
    //   B(t) | K(t+1), V(t) start loading  | stencil and softmax of t -> P(t)
    // The first key tile (no shared column block, no P.V yet) is its own copy
    // of the step, so that the loop holds only the steady-state forms.
    auto step = [&](const int t, auto first_t) {
        constexpr bool FIRST = decltype(first_t)::value;
        const int j0 = t * BN;
        const bool cur = t <= qt;
        barrier_lds();  // A: K(t), V(t-1) in LDS (each wave waited for its DMA); P(t-1) published

        // logit tiles: own row block of head hs (five column blocks), then a
        // share of the halo blocks; the fragments of the next block are read
        // before the products of the current one
        // REUSE (every key tile after the first): column block 0 of the tile
        // (keys j0 - XL .. j0 - XL + 15) is column block 4 of the previous
        // tile, copied into place before the logit products; only blocks 1..4
        // are computed, and the eight halo blocks (both heads) are one per wave
        auto logits = [&](auto masked, auto reuse) {
            constexpr bool M = decltype(masked)::value, R = decltype(reuse)::value;
            constexpr int CB0 = R ? 1 : 0;
            const bf16_t *kh = kbuf + hs * KROWS * D + l16 * D;
            auto kload = [&](QFrag<D> &f, const bf16_t *rows, int cb) {
#pragma unroll
                for (int t = 0; t < 4; ++t) f.x[t] = *reinterpret_cast<const bf16x8 *>(rows + 16 * cb * D + koff[t]);
            };
            // the (first) halo block of this wave: head hh, column block hcb
            const int hh = R ? (wave >> 2) : (wave / NCB);
            const int hcb = R ? 1 + (wave & 3) : (wave % NCB);
            QFrag<D> kf[2], hq, hk;
            kload(kf[CB0 & 1], kh, CB0);
            u32x2 prev;  // converted block waiting for its store partner
#pragma unroll
            for (int cb = CB0; cb < NCB; ++cb) {
                if (cb + 1 < NCB) {
                    kload(kf[(cb + 1) & 1], kh, cb + 1);
                } else if (CQ > 1) {
                    kload(hk, kbuf + fresh((hh * KROWS + 16 * hcb + l16) * D), 0);
                }
                // raw logits, or (POST) probabilities with the row's statistics
                u32x2 v;
                if constexpr (POST) {
                    v = cvt_prob<M>(1 + rw, cb, qk(kf[cb & 1], qown), i0, j0, XL, T, pm_o, pil_o, p.sc, lane);
                } else {
                    f32x4 xs;
                    v = cvt_block<M>(1 + rw, cb, qk(kf[cb & 1], qown), i0, j0, XL, T, EXACT, lane, xs);
                    if (cb == 0)
                        store_centre<0, !PP>(crow, xs, v, t, lane);
                    else if (cb == NCB - 1)
                        store_centre<NCB - 1, !PP>(crow, xs, v, t, lane);
                    else
                        store_centre<1, !PP>(reinterpret_cast<unsigned char *>(crow) + 16 * (cb - 1) * (PP ? 2 : 4),
                                               xs, v, t, lane);
                }
                if ((cb - CB0) & 1)
                    store_pair<CQ>(xo, 1 + rw, cb - 1, prev, xo, 1 + rw, cb, v, lane);
                else
                    prev = v;
            }
            if (CQ > 1) {
                // halo blocks: with REUSE one per wave; else q = wave and, for waves 0
                // and 1, q = wave + 8 (q = h * NCB + cb), the first stored with the
                // last own block
                kload(hq, qhbuf + fresh((hh * HALO + l16) * D), 0);
                u32x2 v;
                f32x4 nores;  // halo rows: not in the centre-tap plane
                if constexpr (POST)
                    v = cvt_prob<M>(0, hcb, qk(hk, hq), i0, j0, XL, T, R ? pm_h : stm[hh * EXT_R + l16],
                                    R ? pil_h : stil[hh * EXT_R + l16], p.sc, lane);
                else
                    v = cvt_block<M>(0, hcb, qk(hk, hq), i0, j0, XL, T, EXACT, lane, nores);
                f16_t *xhh = xbuf + hh * EXT_R * XP;
                if (R) {
                    store_pair<CQ>(xhh, 0, hcb, v, xhh, 0, hcb, v, lane, true);
                } else {
                    store_pair<CQ>(xo, 1 + rw, NCB - 1, prev, xhh, 0, hcb, v, lane);
                    if (wave + 8 < CH * NCB) {
                        const int h = (wave + 8) / NCB, hc = (wave + 8) % NCB;
                        kload(hq, qhbuf + fresh((h * HALO + l16) * D), 0);
                        kload(hk, kbuf + fresh((h * KROWS + 16 * hc + l16) * D), 0);
                        u32x2 v2;
                        if constexpr (POST)
                            v2 = cvt_prob<M>(0, hc, qk(hk, hq), i0, j0, XL, T, stm[h * EXT_R + l16],
                                             stil[h * EXT_R + l16], p.sc, lane);
                        else
                            v2 = cvt_block<M>(0, hc, qk(hk, hq), i0, j0, XL, T, EXACT, lane, nores);
                        f16_t *xh2 = xbuf + h * EXT_R * XP;
                        store_pair<CQ>(xh2, 0, hc, v2, xh2, 0, hc, v2, lane, true);
                    }
                }
            } else if (!R) {
                store_pair<CQ>(xo, 1 + rw, NCB - 1, prev, xo, 1 + rw, NCB - 1, prev, lane, true);
            }
        };
        if constexpr (!FIRST) {
            // P.V of tile t - 1 (ahead of the logit products of t in program
            // order; the two touch disjoint buffers): bring the accumulators
            // into the frame of its maxima first
            const int tp = t - 1;
#pragma unroll
            for (int s = 0; s < CH; ++s) {
                if (tp > 0 && fl[s * 4 + rw]) {
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) f[r] = al[s * BM + 16 * rw + 4 * g4 + r];
#pragma unroll
                    for (int a = 0; a < CH; ++a) {
                        if (DIAG && a != s) continue;  // no head mix: only U[a][a]
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                            for (int r = 0; r < 4; ++r) U[s][a][nb][r] *= f[r];
                    }
                }
            }
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                bf16x8 av[CH], avl[CH];
#pragma unroll
                for (int s = 0; s < CH; ++s) {
                    av[s] = pbuf[((s * 4 + rw) * 2 + cs) * 64 + lane];
                    if (PP) avl[s] = pbuf[CH * 4 * 2 * 64 + ((s * 4 + rw) * 2 + cs) * 64 + lane];
                }
                const int kb0 = 32 * cs + 4 * g4;  // keys of slots 0-3 and 4-7, in the producing lanes' order
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                    for (int a = 0; a < CH; ++a) {
                        const bf16_t *va = vbuf + a * BN * D;
                        const tile::s16x4 u0 = vread_tr4(va, kb0, dbase + 16 * nb, l16);
                        const tile::s16x4 u1 = vread_tr4(va, kb0 + 16, dbase + 16 * nb, l16);
                        typedef short s16x8 __attribute__((ext_vector_type(8)));
                        const s16x8 u = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                        const bf16x8 bv = __builtin_bit_cast(bf16x8, u);
#pragma unroll
                        for (int s = 0; s < CH; ++s) {
                            if (DIAG && s != a) continue;
                            if constexpr (F16PV)
                                U[s][a][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    __builtin_bit_cast(f16x8, av[s]), __builtin_bit_cast(f16x8, bv), U[s][a][nb], 0, 0, 0);
                            else
                                U[s][a][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s], bv, U[s][a][nb], 0, 0, 0);
                            // P kept to ~16 bits: the remainder's product
                            if (PP)
                                U[s][a][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(avl[s], bv, U[s][a][nb], 0, 0, 0);
                        }
                    }
            }
        }
        // key tiles whose logit blocks (halo rows included) are all inside
        // [0, T) and, with Mask_0, all in the past of every row: no masks
        const int kfirst = j0 - XL, klast = j0 - XL + 16 * NCB - 1;
        const bool inner = kfirst >= 0 && i0 >= HALO && i0 + BM <= T && (EXACT ? klast < T : klast <= i0 - HALO);
        if (!FIRST && cur) {
            // column block 4 of tile t-1 is column block 0 of tile t: 16-byte
            // chunks 8, 9 -> 0, 1 (which keeps the row swizzle), each wave for the
            // rows whose block 4 it writes next (own rows; halo rows: the waves of
            // halo column block 4), so its own program order keeps the read first
            if (lane < 32) {
                f16_t *rp = xo + (HALO + 16 * rw + (lane >> 1)) * XP;
                *reinterpret_cast<u32x4 *>(rp + 8 * (lane & 1)) =
                    *reinterpret_cast<const u32x4 *>(rp + 8 * (8 + (lane & 1)));
            } else if (CQ > 1 && (wave & 3) == 3) {
                f16_t *rp = xbuf + (wave >> 2) * EXT_R * XP + ((lane - 32) >> 1) * XP;
                *reinterpret_cast<u32x4 *>(rp + 8 * (lane & 1)) =
                    *reinterpret_cast<const u32x4 *>(rp + 8 * (8 + (lane & 1)));
            }
        }
        if (cur) {
            if constexpr (!FIRST) {
                if (inner)
                    logits(std::false_type{}, std::true_type{});
                else
                    logits(std::true_type{}, std::true_type{});
            } else {
                if (inner)
                    logits(std::false_type{}, std::false_type{});
                else
                    logits(std::true_type{}, std::false_type{});
            }
        }
        barrier_lds();  // B: logit tiles of t published; K, V and probability buffers free
        if (t < qt) dma_pair<false, KROWS>(kbuf, K, hstride, j0 + BN - XL, T, wave, lane);  // K(t+1)
        if (cur) dma_pair<true, BN>(vbuf, V, hstride, j0, T, wave, lane);                      // V(t)

        if (cur) {
            float c[16];
            const int par = (t & 1) ? 64 : 0;  // this key tile's column of keys 0..7 in the centre-tap plane
            if constexpr (C3D)
                stencil64_pair<CQ>(xo, xbuf + (1 - hs) * EXT_R * XP, rho, tf, tfo, crow, par, c00, lane, c);
            else if (EXACT && j0 - XL + 79 > i0 + 16 * rw)
                stencil64<CQ, true, CORR>(xo, rho, tf, qabs - (j0 - XL + 8 * g4), crow, par, c00, lane, c);
            else
                stencil64<CQ, false, CORR>(xo, rho, tf, 0, crow, par, c00, lane, c);
            if constexpr (POST) {
                // Mask_0 after the convolution (only the diagonal tile has keys in
                // the future of its rows); no renormalisation
                if (t == qt) {
#pragma unroll
                    for (int o = 0; o < 16; ++o) {
                        const int key = 16 * (o >> 2) + 4 * g4 + (o & 3);
                        c[o] = (j0 + key <= qabs) ? c[o] : 0.f;
                    }
                }
                bf16x8 v8[2], v8l[2];
#pragma unroll
                for (int o = 0; o < 16; ++o) {
                    v8[o >> 3][o & 7] = (bf16_t)c[o];
                    if (PP) v8l[o >> 3][o & 7] = (bf16_t)(c[o] - (float)v8[o >> 3][o & 7]);
                }
                if constexpr (F16PV) {
                    f16x8 h8[2];
#pragma unroll
                    for (int o = 0; o < 16; ++o) h8[o >> 3][o & 7] = (f16_t)f16_range(c[o]);
                    v8[0] = __builtin_bit_cast(bf16x8, h8[0]);
                    v8[1] = __builtin_bit_cast(bf16x8, h8[1]);
                }
                pbuf[((hs * 4 + rw) * 2 + 0) * 64 + lane] = v8[0];
                pbuf[((hs * 4 + rw) * 2 + 1) * 64 + lane] = v8[1];
                if (PP) {
                    pbuf[CH * 4 * 2 * 64 + ((hs * 4 + rw) * 2 + 0) * 64 + lane] = v8l[0];
                    pbuf[CH * 4 * 2 * 64 + ((hs * 4 + rw) * 2 + 1) * 64 + lane] = v8l[1];
                }
                if (lane == 0) fl[hs * 4 + rw] = 0;  // no rescale
            } else {
                // Mask_-inf (only the diagonal tile has keys in the future of its
                // rows), the row maximum over the 64 keys, probabilities
                if (t == qt) {
#pragma unroll
                    for (int o = 0; o < 16; ++o) {
                        const int key = 16 * (o >> 2) + 4 * g4 + (o & 3);
                        c[o] = (j0 + key <= qabs) ? c[o] : NEG_INF;
                    }
                }
                float mx = NEG_INF;
#pragma unroll
                for (int o = 0; o < 16; ++o) mx = fmaxf(mx, c[o]);
                mx = row_max4(mx);
                // every row has a causal key in tile 0, so m_new is finite
                const float m_new = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                m_run = m_new;
                float ls = 0.f;
                bf16x8 v8[2], v8l[2];
                f16x8 h8[2];
#pragma unroll
                for (int o = 0; o < 16; ++o) {
                    const float e = __builtin_amdgcn_exp2f(c[o] - m_new);  // exp2(-inf) = 0 in the future
                    ls += e;
                    if constexpr (F16PV) {
                        h8[o >> 3][o & 7] = (f16_t)e;  // in [0, 1]
                    } else {
                        v8[o >> 3][o & 7] = (bf16_t)e;
                        if (PP) v8l[o >> 3][o & 7] = (bf16_t)(e - (float)v8[o >> 3][o & 7]);
                    }
                }
                if constexpr (F16PV) {
                    v8[0] = __builtin_bit_cast(bf16x8, h8[0]);
                    v8[1] = __builtin_bit_cast(bf16x8, h8[1]);
                }
                l_run = __builtin_fmaf(l_run, alpha, ls);
                pbuf[((hs * 4 + rw) * 2 + 0) * 64 + lane] = v8[0];
                pbuf[((hs * 4 + rw) * 2 + 1) * 64 + lane] = v8[1];
                if (PP) {
                    pbuf[CH * 4 * 2 * 64 + ((hs * 4 + rw) * 2 + 0) * 64 + lane] = v8l[0];
                    pbuf[CH * 4 * 2 * 64 + ((hs * 4 + rw) * 2 + 1) * 64 + lane] = v8l[1];
                }
                if (g4 == 0) al[hs * BM + io] = alpha;
                const bool moved = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
                if (lane == 0) fl[hs * 4 + rw] = moved ? 1 : 0;
            }
            wait_vm_all();  // K(t+1) and V(t) have landed
            // F16PV: this wave's own V pieces to fp16 in place (published, with
            // the other waves', by the next barrier)
            if constexpr (F16PV) v_to_f16<BN>(vbuf, wave, lane);
        }
        };
    step(0, std::true_type{});
    for (int t = 1; t <= qt + 1; ++t) step(t, std::false_type{});

    // row sums l_b -> 1/l_b in al (after every wave's last P.V read of al);
    // POST: the probabilities were normalised before the convolution
    const float lsum = row_sum4(l_run);
    __syncthreads();
    if (g4 == 0) al[hs * BM + io] = POST ? 1.0f : 1.0f / lsum;
    __syncthreads();

    // O^a = sum_b w_ab U_{b,a} / l_b  (rows 16rw + 4g4 + r, d-columns dbase + 16nb + l16)
    f32x4 acc[CH][4];
    {
        float il[CH][4];
#pragma unroll
        for (int s = 0; s < CH; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) il[s][r] = al[s * BM + 16 * rw + 4 * g4 + r];
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float o = 0.f;
#pragma unroll
                    for (int s = 0; s < CH; ++s)
                        if (!DIAG || s == a) o = __builtin_fmaf(w_s[a * CH + s] * il[s][r], U[s][a][nb][r], o);
                    acc[a][nb][r] = o;
                }
    }

    if constexpr (PREP) {
        // ---------- epilogue of the gradient preparation (instead of the output) ----------
        // row statistics of head hs for row io: log2-domain maximum and 1/sum
        if (g4 == 0 && qabs < T) {
            const size_t ri = ((size_t)b * p.H + h0 + hs) * T + qabs;
            pa.ws_m[ri] = m_run;
            pa.ws_il[ri] = 1.0f / lsum;
        }
        float *ep = reinterpret_cast<float *>(smem + lay.x_off);  // the logit tiles are free now
        float *red = ep;                                          // [rw][a][dgamma, dbeta][D]
        float *sx = red + 4 * CH * 2 * D;                         // [half][a][s1, s2][row]
        float *gred = sx + 2 * CH * 2 * BM;                       // [wave][a]
        float *dx = gred + 8 * CH;                                // [half][s][row]
        auto half_sum = [&](float v) {
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            return v;
        };
        // GroupNorm statistics over d (two d halves through LDS)
        float mu[CH][4], rstd[CH][4];
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sum = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) sum += acc[a][nb][r];
                sum = half_sum(sum);
                if (l16 == 0) gnx[(hs * CH + a) * BM + 16 * rw + 4 * g4 + r] = sum;
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
                for (int nb = 0; nb < 4; ++nb) {
                    const float dl = acc[a][nb][r] - mu[a][r];
                    v2s = __builtin_fmaf(dl, dl, v2s);
                }
                v2s = half_sum(v2s);
                if (l16 == 0) gnx[(hs * CH + a) * BM + 16 * rw + 4 * g4 + r] = v2s;
            }
        __syncthreads();
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rw + 4 * g4 + r;
                const float var = (gnx[(0 * CH + a) * BM + row] + gnx[(1 * CH + a) * BM + row]) * (1.0f / D);
                rstd[a][r] = 1.0f / __builtin_sqrtf(var + p.eps);
            }
        // GroupNorm backward: dxh = dY * s_a * gamma; dO = rstd (dxh - mean(dxh) - xh mean(dxh xh))
        const bf16_t *dY = pa.dout;
        float dgw[CH][4], dgb[CH][4], gpart[CH], dxh[CH][4][4], xh[CH][4][4];
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            const int h = h0 + a;
            const float *gw = p.gn_w + (size_t)h * D;
            const float *gb = p.gn_b + (size_t)h * D;
            const float sa = head_factor(p, h);
            gpart[a] = 0.f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) dgw[a][nb] = dgb[a][nb] = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i0 + 16 * rw + 4 * g4 + r;
                float s1 = 0.f, s2 = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int col = dbase + 16 * nb + l16;
                    xh[a][nb][r] = (acc[a][nb][r] - mu[a][r]) * rstd[a][r];
                    const float dy = row < T ? (float)dY[((size_t)b * p.H + h) * hstride + (size_t)row * D + col] : 0.f;
                    const float dys = dy * sa;
                    dgb[a][nb] += dys;
                    dgw[a][nb] = __builtin_fmaf(dys, xh[a][nb][r], dgw[a][nb]);
                    gpart[a] = __builtin_fmaf(dy, xh[a][nb][r] * gw[col] + gb[col], gpart[a]);
                    dxh[a][nb][r] = dys * gw[col];
                    s1 += dxh[a][nb][r];
                    s2 = __builtin_fmaf(dxh[a][nb][r], xh[a][nb][r], s2);
                }
                s1 = half_sum(s1);
                s2 = half_sum(s2);
                if (l16 == 0) {
                    sx[((hs * CH + a) * 2 + 0) * BM + 16 * rw + 4 * g4 + r] = s1;
                    sx[((hs * CH + a) * 2 + 1) * BM + 16 * rw + 4 * g4 + r] = s2;
                }
            }
            // dgamma, dbeta of this wave's 16 rows: the four lane groups, then the waves via LDS
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                float u = dgw[a][nb], t = dgb[a][nb];
                u += __shfl_xor(u, 16);
                u += __shfl_xor(u, 32);
                t += __shfl_xor(t, 16);
                t += __shfl_xor(t, 32);
                if (g4 == 0) {
                    red[((rw * CH + a) * 2 + 0) * D + dbase + 16 * nb + l16] = u;
                    red[((rw * CH + a) * 2 + 1) * D + dbase + 16 * nb + l16] = t;
                }
            }
            float gsum = gpart[a];
#pragma unroll
            for (int sh = 1; sh < 64; sh <<= 1) gsum += __shfl_xor(gsum, sh);
            const float sg = p.gate ? 1.0f / (1.0f + __expf(-p.gate[h])) : 1.0f;
            if (lane == 0) gred[wave * CH + a] = gsum * p.depth_scale * sg * (1.0f - sg);
        }
        __syncthreads();
        for (int i = tid; i < CH * 2 * D; i += NT) {
            const int a = i / (2 * D), which = (i / D) % 2, col = i % D;
            float t = 0.f;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) t += red[((w4 * CH + a) * 2 + which) * D + col];
            atomicAdd((which ? pa.dgn_b : pa.dgn_w) + (size_t)(h0 + a) * D + col, t);
        }
        if (p.gate && tid < CH) {
            float t = 0.f;
#pragma unroll
            for (int w8 = 0; w8 < 8; ++w8) t += gred[w8 * CH + tid];
            atomicAdd(pa.dgate + h0 + tid, t);
        }
        // dO (bf16 high part and remainder), then D^s_i = sum_a w_as dO^a_i . (P^s V^a)_i
        float dOr[CH][4][4];
#pragma unroll
        for (int a = 0; a < CH; ++a) {
            const int h = h0 + a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rowt = 16 * rw + 4 * g4 + r, row = i0 + rowt;
                const float s1 = (sx[((0 * CH + a) * 2 + 0) * BM + rowt] + sx[((1 * CH + a) * 2 + 0) * BM + rowt]) *
                                 (1.0f / D);
                const float s2 = (sx[((0 * CH + a) * 2 + 1) * BM + rowt] + sx[((1 * CH + a) * 2 + 1) * BM + rowt]) *
                                 (1.0f / D);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const float dox = rstd[a][r] * (dxh[a][nb][r] - s1 - xh[a][nb][r] * s2);
                    if (row < T) {
                        const size_t at = ((size_t)b * p.H + h) * hstride + (size_t)row * D + dbase + 16 * nb + l16;
                        const bf16_t dh = (bf16_t)dox;
                        pa.ws_dO[at] = dh;
                        pa.ws_dOl[at] = (bf16_t)(dox - (float)dh);
                    }
                    dOr[a][nb][r] = row < T ? dox : 0.f;
                }
            }
        }
        float il[CH][4];
#pragma unroll
        for (int s = 0; s < CH; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) il[s][r] = al[s * BM + 16 * rw + 4 * g4 + r];
#pragma unroll
        for (int s = 0; s < CH; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float t = 0.f;
#pragma unroll
                for (int a = 0; a < CH; ++a) {
                    float u = 0.f;
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) u = __builtin_fmaf(dOr[a][nb][r], U[s][a][nb][r], u);
                    t = __builtin_fmaf(w_s[a * CH + s], u, t);
                }
                t = half_sum(t * il[s][r]);
                if (l16 == 0) dx[(hs * CH + s) * BM + 16 * rw + 4 * g4 + r] = t;
            }
        __syncthreads();
        if (hs == 0 && l16 == 0) {
#pragma unroll
            for (int s = 0; s < CH; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rowt = 16 * rw + 4 * g4 + r, row = i0 + rowt;
                    if (row < T)
                        pa.ws_D[((size_t)b * p.H + h0 + s) * T + row] =
                            dx[(0 * CH + s) * BM + rowt] + dx[(1 * CH + s) * BM + rowt];
                }
        }
        return;
    }

    if constexpr (QUAD) {
        // the first sweep stores its share, each later one adds the stored
        // sum, and all but the last store the new sum (float32 throughout, so
        // that mixing weights which cancel keep the precision of one sweep)
        const bool last = pi + 1 == p.npair;
#pragma unroll
        for (int a = 0; a < CH; ++a)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = (a * 4 + nb) * 4 + r;
                    if (pi > 0) acc[a][nb][r] += keep[i];
                    if (!last) keep[i] = acc[a][nb][r];
                }
        if (!last) {
            ++pi;
            __syncthreads();  // every wave is done with this sweep's LDS
            goto sweep;
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
            for (int nb = 0; nb < 4; ++nb) sum += acc[a][nb][r];
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            sum += __shfl_xor(sum, 8);
            if (l16 == 0) gnx[(hs * CH + a) * BM + 16 * rw + 4 * g4 + r] = sum;
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
            for (int nb = 0; nb < 4; ++nb) {
                const float dl = acc[a][nb][r] - mu[a][r];
                v2s = __builtin_fmaf(dl, dl, v2s);
            }
            v2s += __shfl_xor(v2s, 1);
            v2s += __shfl_xor(v2s, 2);
            v2s += __shfl_xor(v2s, 4);
            v2s += __shfl_xor(v2s, 8);
            if (l16 == 0) gnx[(hs * CH + a) * BM + 16 * rw + 4 * g4 + r] = v2s;
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
                for (int nb = 0; nb < 4; ++nb) {
                    const int col = dbase + 16 * nb + l16;
                    const float y = ((acc[a][nb][r] - mu[a][r]) * rstd * gw[col] + gb[col]) * hf;
                    dst[col] = (bf16_t)y;
                }
            }
        }
    }
}

template <int CQ, int CK, bool EXACT, bool POST = false, bool C3D = false, bool NOMIX = false, bool QUAD = false,
          bool F16PV = false>
hipError_t launch(const Params &p, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_v4<CQ, CK, EXACT, false, POST, C3D, NOMIX, QUAD, F16PV>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p, PrepArgs{});
    return hipGetLastError();
}

template <int CQ, int CK, bool EXACT>
hipError_t launch_prep(const Params &p, const PrepArgs &pa, int grid, size_t lds, hipStream_t s)
{
    auto fn = mta_fwd_v4<CQ, CK, EXACT, true>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, s, p, pa);
    return hipGetLastError();
}

}  // namespace v4
}  // namespace mta
