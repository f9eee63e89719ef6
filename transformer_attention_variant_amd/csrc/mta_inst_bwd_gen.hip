// The backward pass for every placement (mta_bwd_gen.h): the slot plan, the
// chunk loop over head groups and the launch sequence.
#include "mta_bwd_gen.h"
#include "mta_bwd.h"

namespace mta {
namespace gen {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int tiles_per_side(int T) { return (T + TB - 1) / TB; }

// Which workspace slot holds each map.  A map that nothing reads after the
// stage that replaces it shares its slot with the replacement:
//   C  = S when no key-query convolution precedes the softmax;
//   L  = C unless a head mix precedes it (then L has its own slot, since the
//        mix's gradient needs C);
//   P  = L (the softmax runs in place: the backward needs no L);
//   P2 = P unless a convolution follows the softmax;
//   P3 = P2 unless a head mix follows it;
//   two gradient slots, used alternately.
struct Slots {
    int S, C, L, P, P2, P3, g1, g2, n;
};

Slots plan(int kq_place, int head_place)
{
    Slots s;
    int next = 0;
    s.S = next++;
    s.C = kq_place != KQ_POST ? next++ : s.S;
    s.L = head_place == KQ_PRE ? next++ : s.C;
    s.P = s.L;
    s.P2 = kq_place == KQ_POST ? next++ : s.P;
    s.P3 = head_place == KQ_POST ? next++ : s.P2;
    s.g1 = next++;
    s.g2 = next++;
    s.n = next;
    return s;
}

#define GEN_CHECK()                                \
    do {                                           \
        const hipError_t e_ = hipGetLastError();   \
        if (e_ != hipSuccess) return e_;           \
    } while (0)

template <int CH>
hipError_t mix_fwd(const GParams &p, const float *in, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(gen_mix_fwd<CH>, dim3(p.n_band, p.nu), dim3(NTH), 0, s, p, in, out);
    return hipGetLastError();
}

template <int CH>
hipError_t mix_bwd(const GParams &p, float *g, const float *in, hipStream_t s)
{
    hipLaunchKernelGGL(gen_mix_bwd<CH>, dim3(p.n_band, p.nu), dim3(NTH), 0, s, p, g, in);
    return hipGetLastError();
}

template <int CH>
hipError_t mix_fwd_wide(const GParams &p, const float *in, float *out, hipStream_t s)
{
    hipLaunchKernelGGL(gen_mix_fwd_wide<CH>, dim3(p.n_band, p.nu), dim3(NTH), 0, s, p, in, out);
    return hipGetLastError();
}

// dw first (it reads the gradient slot), then the in-place transform
template <int CH>
hipError_t mix_bwd_wide(const GParams &p, float *g, const float *in, hipStream_t s)
{
    hipLaunchKernelGGL(gen_mix_dw_wide<CH>, dim3(p.n_band, p.nu, CH), dim3(NTH), 0, s, p, g, in);
    GEN_CHECK();
    hipLaunchKernelGGL(gen_mix_bwd_wide<CH>, dim3(p.n_band, p.nu), dim3(NTH), 0, s, p, g);
    return hipGetLastError();
}

hipError_t mix(bool fwd, const GParams &p, const float *in, float *out, hipStream_t s)
{
    switch (p.c_h) {
    case 1: return fwd ? mix_fwd<1>(p, in, out, s) : mix_bwd<1>(p, out, in, s);
    case 2: return fwd ? mix_fwd<2>(p, in, out, s) : mix_bwd<2>(p, out, in, s);
    case 4: return fwd ? mix_fwd<4>(p, in, out, s) : mix_bwd<4>(p, out, in, s);
    case 8: return fwd ? mix_fwd_wide<8>(p, in, out, s) : mix_bwd_wide<8>(p, out, in, s);
    case 16: return fwd ? mix_fwd_wide<16>(p, in, out, s) : mix_bwd_wide<16>(p, out, in, s);
    default: return hipErrorInvalidValue;
    }
}

// Launches a stencil kernel with its dynamic LDS (above 64 KB for large c_q).
template <typename... A>
hipError_t launch_conv(void (*k)(GParams, A...), dim3 grid, size_t lds, hipStream_t s, const GParams &p,
                       A... args)
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, dim3(NTH), lds, s, p, args...);
    return hipGetLastError();
}

#define GEN_TRY(x)                      \
    do {                                \
        const hipError_t e_ = (x);      \
        if (e_ != hipSuccess) return e_; \
    } while (0)

template <typename DT, int D>
hipError_t run_chunk(const GParams &p, float *const *slot, const Slots &sl, hipStream_t s)
{
    const size_t lds1 = conv_lds_bytes(p.c_q, 1), lds2 = conv_lds_bytes(p.c_q, 2);
    const int heads = p.nu * p.c_h;
    const dim3 band(p.n_band, heads), rows_t(p.nt, heads), rows4(p.Tp / 4, heads);
    const dim3 blk(NTH);
    const int kq = p.kq_place, hp = p.head_place;
    const int cmode = kq == KQ_EXACT ? M_EXACT : M_PRE;

    // forward: S, C, L, P, P2, P3, O
    constexpr bool B16 = std::is_same<DT, bf16_t>::value;  // bf16 inputs: the 16-bit products
    if constexpr (B16)
        hipLaunchKernelGGL((gen_gemm_nt16<D, SRC_TENSOR>), band, blk, 0, s, p, p.q, p.k, slot[sl.S], p.inv_sqrt_d);
    else
        hipLaunchKernelGGL((gen_gemm_nt<DT, D, SRC_TENSOR>), band, blk, 0, s, p, p.q, p.k, slot[sl.S], p.inv_sqrt_d);
    GEN_CHECK();
    if (kq != KQ_POST) {
        const float *in = slot[sl.S];
        if (cmode == M_EXACT)
            GEN_TRY(launch_conv(gen_conv_fwd<M_EXACT>, band, lds1, s, p, in, slot[sl.C]));
        else
            GEN_TRY(launch_conv(gen_conv_fwd<M_PRE>, band, lds1, s, p, in, slot[sl.C]));
    }
    if (hp == KQ_PRE) {
        const hipError_t e = mix(true, p, slot[sl.C], slot[sl.L], s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gen_softmax_fwd, rows4, blk, 0, s, p, slot[sl.P]);
    GEN_CHECK();
    if (kq == KQ_POST) {
        const float *in = slot[sl.P];
        GEN_TRY(launch_conv(gen_conv_fwd<M_POST>, band, lds1, s, p, in, slot[sl.P2]));
    }
    if (hp == KQ_POST) {
        const hipError_t e = mix(true, p, slot[sl.P2], slot[sl.P3], s);
        if (e != hipSuccess) return e;
    }
    if constexpr (B16)
        hipLaunchKernelGGL((gen_gemm_mn16<D, true>), rows_t, blk, 0, s, p, slot[sl.P3], p.v, nullptr, 1.0f);
    else
        hipLaunchKernelGGL((gen_gemm_mn<DT, D, true>), rows_t, blk, 0, s, p, slot[sl.P3], p.v, nullptr, 1.0f);
    GEN_CHECK();

    // backward
    hipLaunchKernelGGL((gen_groupnorm_bwd<DT, D>), dim3((p.T + 63) / 64, heads), blk, 0, s, p);
    GEN_CHECK();
    hipLaunchKernelGGL((gen_gemm_tn<DT, D, SRC_OBUF>), rows_t, blk, 0, s, p, slot[sl.P3], nullptr, p.dv, 1.0f);
    GEN_CHECK();
    if constexpr (B16)
        hipLaunchKernelGGL((gen_gemm_nt16<D, SRC_OBUF>), band, blk, 0, s, p, nullptr, p.v, slot[sl.g1], 1.0f);
    else
        hipLaunchKernelGGL((gen_gemm_nt<DT, D, SRC_OBUF>), band, blk, 0, s, p, nullptr, p.v, slot[sl.g1], 1.0f);
    GEN_CHECK();
    int cur = sl.g1, other = sl.g2;
    if (hp == KQ_POST) {  // dP3 -> dP2, dw
        const hipError_t e = mix(false, p, slot[sl.P2], slot[cur], s);
        if (e != hipSuccess) return e;
    }
    if (kq == KQ_POST) {  // dP2 -> dP, dtheta
        const float *g = slot[cur], *in = slot[sl.P];
        GEN_TRY(launch_conv(gen_conv_bwd<M_POST>, band, lds2, s, p, g, in, slot[other]));
        const int t = cur;
        cur = other;
        other = t;
    }
    hipLaunchKernelGGL(gen_softmax_bwd, rows4, blk, 0, s, p, slot[sl.P], slot[cur]);
    GEN_CHECK();
    if (hp == KQ_PRE) {  // dL -> dC, dw
        const hipError_t e = mix(false, p, slot[sl.C], slot[cur], s);
        if (e != hipSuccess) return e;
    }
    if (kq != KQ_POST) {  // dC -> dS, dtheta
        const float *g = slot[cur], *in = slot[sl.S];
        if (cmode == M_EXACT)
            GEN_TRY(launch_conv(gen_conv_bwd<M_EXACT>, band, lds2, s, p, g, in, slot[other]));
        else
            GEN_TRY(launch_conv(gen_conv_bwd<M_PRE>, band, lds2, s, p, g, in, slot[other]));
        const int t = cur;
        cur = other;
        other = t;
    }
    if constexpr (B16) {
        hipLaunchKernelGGL((gen_gemm_mn16<D, false>), rows_t, blk, 0, s, p, slot[cur], p.k, p.dq, p.inv_sqrt_d);
        GEN_CHECK();
        hipLaunchKernelGGL((gen_gemm_tn16<D>), rows_t, blk, 0, s, p, slot[cur], p.q, p.dk, p.inv_sqrt_d);
    } else {
        hipLaunchKernelGGL((gen_gemm_mn<DT, D, false>), rows_t, blk, 0, s, p, slot[cur], p.k, p.dq, p.inv_sqrt_d);
        GEN_CHECK();
        hipLaunchKernelGGL((gen_gemm_tn<DT, D, SRC_TENSOR>), rows_t, blk, 0, s, p, slot[cur], p.q, p.dk,
                           p.inv_sqrt_d);
    }
    GEN_CHECK();
    return hipSuccess;
}

template <typename DT>
hipError_t run_chunk_d(const GParams &p, float *const *slot, const Slots &sl, hipStream_t s)
{
    switch (p.d) {
    case 32: return run_chunk<DT, 32>(p, slot, sl, s);
    case 64: return run_chunk<DT, 64>(p, slot, sl, s);
    case 128: return run_chunk<DT, 128>(p, slot, sl, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int n_slots(int kq_place, int head_place) { return plan(kq_place, head_place).n; }

size_t unit_bytes(int T, int d, int c_h, int kq_place, int head_place)
{
    const size_t Tp = (size_t)tiles_per_side(T) * TB;
    return (size_t)n_slots(kq_place, head_place) * align256((size_t)c_h * Tp * Tp * 4) +
           align256((size_t)c_h * T * d * 4);
}

size_t workspace_bytes(int B, int H, int T, int d, int c_h, int kq_place, int head_place)
{
    const size_t ub = unit_bytes(T, d, c_h, kq_place, head_place);
    const size_t units = (size_t)B * (H / c_h);
    size_t n = CHUNK_CAP / ub;
    if (n < 1) n = 1;
    if (n > units) n = units;
    if (n > (size_t)(65535 / c_h)) n = 65535 / c_h;
    return n * ub;
}

hipError_t backward(const GenArgs &a, void *ws, size_t ws_bytes, hipStream_t s)
{
    GParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
    p.theta = a.theta; p.w = a.w; p.gn_w = a.gn_w; p.gn_b = a.gn_b; p.gate = a.gate;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dtheta = a.dtheta; p.dw = a.dw;
    p.dgn_w = a.dgn_w; p.dgn_b = a.dgn_b; p.dgate = a.dgate;
    p.B = a.B; p.H = a.H; p.T = a.T; p.d = a.d; p.c_q = a.c_q; p.c_k = a.c_k; p.c_h = a.c_h;
    p.G = a.H / a.c_h;
    p.kq_place = a.kq_place; p.head_place = a.head_place;
    p.eps = a.eps; p.depth_scale = a.depth_scale; p.inv_sqrt_d = 1.0f / sqrtf((float)a.d);
    p.nt = tiles_per_side(a.T);
    p.Tp = p.nt * TB;
    p.n_band = p.nt * (p.nt + 1) / 2 + (p.nt - 1);

    const Slots sl = plan(a.kq_place, a.head_place);
    const size_t ub = unit_bytes(a.T, a.d, a.c_h, a.kq_place, a.head_place);
    const int units = a.B * p.G;
    size_t per_chunk = ws_bytes / ub;
    if (per_chunk < 1) return hipErrorInvalidValue;
    if (per_chunk > (size_t)(65535 / a.c_h)) per_chunk = 65535 / a.c_h;

    bwd::ZeroList z{};
    z.p[0] = a.dtheta; z.n[0] = (size_t)a.H * a.c_q * a.c_k;
    z.p[1] = a.dw;     z.n[1] = (size_t)p.G * a.c_h * a.c_h;
    z.p[2] = a.dgn_w;  z.n[2] = (size_t)a.H * a.d;
    z.p[3] = a.dgn_b;  z.n[3] = (size_t)a.H * a.d;
    z.k = 4;
    if (a.dgate) {
        z.p[4] = a.dgate;
        z.n[4] = (size_t)a.H;
        z.k = 5;
    }
    hipError_t e = launch_fill_zero(z, s);
    if (e != hipSuccess) return e;

    for (int u0 = 0; u0 < units; u0 += (int)per_chunk) {
        p.u0 = u0;
        p.nu = units - u0 < (int)per_chunk ? units - u0 : (int)per_chunk;
        // the chunk's slots, then its O buffer, carved from the workspace
        char *base = static_cast<char *>(ws);
        const size_t slot_bytes = align256((size_t)a.c_h * p.Tp * p.Tp * 4) * p.nu;
        float *slot[8];
        for (int k = 0; k < sl.n; ++k) slot[k] = reinterpret_cast<float *>(base + (size_t)k * slot_bytes);
        p.obuf = reinterpret_cast<float *>(base + (size_t)sl.n * slot_bytes);
        e = a.bf16 ? run_chunk_d<bf16_t>(p, slot, sl, s) : run_chunk_d<float>(p, slot, sl, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gen
}  // namespace mta
