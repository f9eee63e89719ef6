// mta_api.hip — the C ABI declared in include/mta.h: host-side validation,
// kernel selection and the asynchronous launch on the caller's stream.
#include <math.h>
#include <stdint.h>
#include <cstring>
#include <mutex>

#include "mta.h"
#include "mta_fwd_v4.h"
#include "mta_fwd_layer.h"
#include "mta_fwd_rep.h"
#include "mta_bwd.h"
#include "mta_bwd_gen_api.h"
#include "mta_launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int validate(const mta_config *c)
{
    if (!c) return MTA_ERR_NULL_ARG;
    if (c->batch < 0 || c->heads < 1 || c->seq_len < 0 || c->head_dim < 1) return MTA_ERR_BAD_SHAPE;
    if (c->c_q < 1 || c->c_k < 1 || c->c_h < 1 || c->heads % c->c_h != 0) return MTA_ERR_BAD_SHAPE;
    if ((c->kq_place != MTA_PRE_SOFTMAX && c->kq_place != MTA_POST_SOFTMAX &&
         c->kq_place != MTA_PRE_SOFTMAX_EXACT) ||
        (c->head_place != MTA_PRE_SOFTMAX && c->head_place != MTA_POST_SOFTMAX))
        return MTA_ERR_BAD_PLACEMENT;
    if (c->dtype != MTA_F32 && c->dtype != MTA_BF16) return MTA_ERR_BAD_DTYPE;
    if (!(c->gn_eps > 0.0f) || !isfinite(c->gn_eps) || !isfinite(c->depth_scale)) return MTA_ERR_BAD_VALUE;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return MTA_ERR_UNSUPPORTED;
    // groups of 8 or 16 heads: the forward on the head-split kernel only (bf16,
    // d = 128, head mix after the softmax; make_plan decides) and the backward
    // with the maps in the workspace
    if (c->c_h != 1 && c->c_h != 2 && c->c_h != 4 && c->c_h != 8 && c->c_h != 16) return MTA_ERR_UNSUPPORTED;
    if (c->c_q > mta::MAX_CQ || c->c_k > mta::MAX_CK) return MTA_ERR_UNSUPPORTED;
    if (c->seq_len > (1 << 24)) return MTA_ERR_UNSUPPORTED;
    // the grid is one workgroup per (batch, head group, 64-row query tile)
    const int64_t n_qt = (c->seq_len + mta::BM - 1) / mta::BM;
    const int64_t grid = n_qt * (int64_t)c->batch * (c->heads / c->c_h);
    if (grid > INT32_MAX) return MTA_ERR_UNSUPPORTED;
    return MTA_OK;
}

size_t lds_bytes(const mta::Params &p, int dtype, int d, int ch)
{
    const int ckp = (p.c_k + 3) & ~3;
    size_t b = (size_t)p.nbuf * mta::EXT_R * p.pitch * 4 + (size_t)2 * ch * mta::EXT_R * 4;
    b += (size_t)((ch * p.c_q * ckp + 3) & ~3) * 4 + (size_t)((ch * ch + 3) & ~3) * 4;
    if (dtype == MTA_BF16) {
        b += d == 32 ? mta::vbuf_bytes<mta::bf16_t, 32>()
                     : d == 64 ? mta::vbuf_bytes<mta::bf16_t, 64>() : mta::vbuf_bytes<mta::bf16_t, 128>();
    } else {
        b += d == 32 ? mta::vbuf_bytes<float, 32>()
                     : d == 64 ? mta::vbuf_bytes<float, 64>() : mta::vbuf_bytes<float, 128>();
    }
    return b;
}

}  // namespace

extern "C" {

int mta_abi_version(void) { return 100; }

const char *mta_status_string(int s)
{
    switch (s) {
    case MTA_OK: return "ok";
    case MTA_ERR_NULL_ARG: return "a required pointer is NULL";
    case MTA_ERR_BAD_SHAPE: return "invalid shape (B,H,T,d, kernel sizes, or H not a multiple of c_h)";
    case MTA_ERR_BAD_PLACEMENT: return "placement must be pre- (0) or post-softmax (1), or exact pre-softmax (2) for kq";
    case MTA_ERR_BAD_DTYPE: return "dtype must be MTA_F32 or MTA_BF16";
    case MTA_ERR_MISALIGNED: return "tensor pointer not aligned (16 bytes for q,k,v,out; 4 for float params)";
    case MTA_ERR_UNSUPPORTED: return "configuration outside the library's limits (d in {32,64,128}, c_h in {1,2,4,8,16}, c_q<=16, c_k<=31, T<=2^24; the forward at c_h 8 or 16: bf16, d=128, head mix after the softmax, c_q x c_k in {1x1,4x9,6x11,8x15})";
    case MTA_ERR_LAUNCH: return "kernel launch failed";
    case MTA_ERR_BAD_VALUE: return "gn_eps must be finite and > 0, depth_scale finite";
    case MTA_ERR_SCRATCH: return "the problem needs more workspace than the library's device scratch array holds";
    default: return "unknown status";
    }
}

// The kernel a valid configuration runs, its launch parameters (shapes and
// tile geometry; the caller fills in the tensor pointers) and its LDS size.
struct Plan {
    mta::LaunchFn fn = nullptr;
    size_t lds = 0;
    int grid = 0;
    const char *name = nullptr;
    mta::Params p{};
};

static int make_plan(const mta_config *cfg, Plan &pl)
{
    const int d = cfg->head_dim, ch = cfg->c_h, cq = cfg->c_q, ck = cfg->c_k;
    const int post = cfg->kq_place == MTA_POST_SOFTMAX;
    const int exact = cfg->kq_place == MTA_PRE_SOFTMAX_EXACT;
    const int hpre = cfg->head_place == MTA_PRE_SOFTMAX;

    mta::Params &p = pl.p;
    p.H = cfg->heads; p.T = cfg->seq_len; p.c_q = cq; p.c_k = ck;
    p.G = cfg->heads / ch;
    p.units = cfg->batch * p.G;
    p.n_qt = (cfg->seq_len + mta::BM - 1) / mta::BM;
    p.head_pre = hpre;
    p.exact = exact;
    p.hl = (ck + 1) / 2 - 1;
    p.ncb = (mta::BN + ck - 1 + 15) / 16;
    p.pitch = p.ncb * 16 + 4;
    p.nbuf = (post && hpre) ? ch : 1;
    p.sc = 1.4426950408889634f / sqrtf((float)d);
    p.eps = cfg->gn_eps;
    p.depth_scale = cfg->depth_scale;
    pl.grid = p.n_qt * p.units;

    constexpr size_t LDS_MAX = 160 * 1024;
    mta::LaunchFn fn = nullptr;
    size_t lds = 0;
    if (cfg->dtype == MTA_BF16) {
        const int ncb0 = p.ncb, pitch0 = p.pitch;
        // the head-split kernel in the form that fits the grouping: c_h = 2 with
        // the head mix after the softmax (one pass with online softmax
        // statistics when the key-query convolution comes before the softmax,
        // two passes when after), the 3D form for the head mix before it, head
        // pairs of single-head groups, four-head groups; else the general kernel
        fn = mta::find_launch_v4(d, ch, cq, ck, post, exact, hpre);
        if (fn) {
            p.ncb = 5;
            p.pitch = p.ncb * 16 + 4;
            lds = (size_t)mta::v4::layout(cq, ck, false, post != 0).total;
            if (lds > LDS_MAX) fn = nullptr;
            else pl.name = post ? "mta_fwd_v4 (two passes, head-split waves, fp16 matrix-core stencil)"
                                : "mta_fwd_v4 (one pass, head-split waves, fp16 matrix-core stencil)";
        }
        if (!fn && hpre && !post && !exact) {
            // head mix before the softmax: by linearity the 3D convolution with
            // kernel w[g][a][b] * theta[b], built in the kernel from both
            fn = mta::find_launch_v4_3d(d, ch, cq, ck);
            if (fn) {
                p.ncb = 5;
                p.pitch = p.ncb * 16 + 4;
                lds = (size_t)mta::v4::layout(cq, ck, false, false, true).total;
                if (lds > LDS_MAX) fn = nullptr;
                else pl.name = "mta_fwd_v4 (one pass, head-split waves, pre-softmax head mix as a 3D convolution, fp16 matrix-core stencil)";
            }
        }
        if (!fn && ch == 1 && !hpre && cfg->heads % 2 == 0) {
            // single-head groups, two per workgroup: the head-split kernel with
            // the 1x1 mix of each head after the softmax (the grid counts head
            // pairs); before the softmax the 1x1 mix scales the logits, which
            // that kernel does not do, so such groups take the general kernel
            fn = mta::find_launch_v4_pairs(d, cq, ck, post, exact);
            if (fn) {
                p.ncb = 5;
                p.pitch = p.ncb * 16 + 4;
                p.G = cfg->heads / 2;
                p.units = cfg->batch * p.G;
                pl.grid = p.n_qt * p.units;
                lds = (size_t)mta::v4::layout(cq, ck, false, post != 0).total;
                if (lds > LDS_MAX) fn = nullptr;
                else pl.name = post ? "mta_fwd_v4 (two passes, head-split waves, head pairs of single-head groups, fp16 matrix-core stencil)"
                                    : "mta_fwd_v4 (one pass, head-split waves, head pairs of single-head groups, fp16 matrix-core stencil)";
            }
            if (!fn) {
                p.G = cfg->heads / ch;
                p.units = cfg->batch * p.G;
                pl.grid = p.n_qt * p.units;
            }
        }
        if (!fn && (ch == 4 || ch == 8 || ch == 16) && !hpre) {
            // groups of four or more heads: the head-split kernel per output
            // head pair, one sweep per source pair (the grid counts output pairs)
            // groups of 8 and 16: P.V with fp16 operands, since the error of
            // one rounding per source head grows with the head mix's
            // cancellation
            const bool f16pv = ch > 4;
            fn = mta::find_launch_v4_quad(d, cq, ck, post, exact, f16pv);
            // the grid counts head pairs, c_h / 2 times the groups validate() bounded
            if ((int64_t)p.n_qt * cfg->batch * (cfg->heads / 2) > INT32_MAX) fn = nullptr;
            if (fn) {
                p.ncb = 5;
                p.pitch = p.ncb * 16 + 4;
                p.G = cfg->heads / 2;
                p.units = cfg->batch * p.G;
                p.npair = ch / 2;
                pl.grid = p.n_qt * p.units;
                lds = (size_t)mta::v4::layout(cq, ck, false, post != 0).total;
                if (lds > LDS_MAX) fn = nullptr;
                else if (ch == 4)
                    pl.name = post ? "mta_fwd_v4 (four-head groups: two source-pair sweeps of two passes, head-split waves, fp16 matrix-core stencil)"
                                   : "mta_fwd_v4 (four-head groups: two source-pair sweeps, head-split waves, fp16 matrix-core stencil)";
                else
                    pl.name = post ? "mta_fwd_v4 (groups of 8 or 16 heads: one source-pair sweep of two passes per head pair, head-split waves, fp16 matrix-core stencil)"
                                   : "mta_fwd_v4 (groups of 8 or 16 heads: one source-pair sweep per head pair, head-split waves, fp16 matrix-core stencil)";
            }
            if (!fn) {
                p.G = cfg->heads / ch;
                p.units = cfg->batch * p.G;
                pl.grid = p.n_qt * p.units;
            }
        }
        if (!fn) {
            p.ncb = ncb0;
            p.pitch = pitch0;
        }
    }
    if (!fn) {
        // the general 4-wave kernel
        fn = cfg->dtype == MTA_BF16 ? mta::find_launch_bf16(d, ch, cq, ck, post, hpre)
                                    : mta::find_launch_f32(d, ch, cq, ck, post, hpre);
        lds = lds_bytes(p, cfg->dtype, d, ch);
        pl.name = "mta_fwd_kernel (two passes, general)";
    }
    if (!fn || lds > LDS_MAX) return MTA_ERR_UNSUPPORTED;
    pl.fn = fn;
    pl.lds = lds;
    return MTA_OK;
}

static int forward_impl(const void *q, const void *k, const void *v, const float *theta_kq,
                        const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                        const mta_config *cfg, void *out, void *stream)
{
    const int vs = validate(cfg);
    if (vs != MTA_OK) return vs;
    if (cfg->batch == 0 || cfg->seq_len == 0) return MTA_OK;  // empty: nothing to do
    if (!q || !k || !v || !theta_kq || !theta_head || !gn_w || !gn_b || !out) return MTA_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(theta_kq) ||
        !aligned4(theta_head) || !aligned4(gn_w) || !aligned4(gn_b) || (gate && !aligned4(gate)))
        return MTA_ERR_MISALIGNED;

    Plan pl;
    const int ps = make_plan(cfg, pl);
    if (ps != MTA_OK) return ps;
    mta::Params &p = pl.p;
    p.q = q; p.k = k; p.v = v;
    p.theta = theta_kq; p.wmix = theta_head; p.gn_w = gn_w; p.gn_b = gn_b; p.gate = gate;
    p.out = out;
    const hipError_t e = pl.fn(p, pl.grid, pl.lds, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
}

int mta_check_config(const mta_config *cfg)
{
    const int vs = validate(cfg);
    if (vs != MTA_OK) return vs;
    // kernel selection and its LDS fit, exactly as mta_forward decides them
    Plan pl;
    return make_plan(cfg, pl);
}

const char *mta_kernel_name(const mta_config *cfg)
{
    if (validate(cfg) != MTA_OK) return nullptr;
    Plan pl;
    return make_plan(cfg, pl) == MTA_OK ? pl.name : nullptr;
}

int mta_forward(const void *q, const void *k, const void *v, const float *theta_kq,
                const float *theta_head, const float *gn_w, const float *gn_b,
                const mta_config *cfg, void *out, void *stream)
{
    return forward_impl(q, k, v, theta_kq, theta_head, gn_w, gn_b, nullptr, cfg, out, stream);
}

int mta_forward_gated(const void *q, const void *k, const void *v, const float *theta_kq,
                      const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                      const mta_config *cfg, void *out, void *stream)
{
    const int vs = validate(cfg);
    if (vs != MTA_OK) return vs;
    if (cfg->batch == 0 || cfg->seq_len == 0) return MTA_OK;
    if (!gate) return MTA_ERR_NULL_ARG;
    return forward_impl(q, k, v, theta_kq, theta_head, gn_w, gn_b, gate, cfg, out, stream);
}

// ---------------------------------------------------------------------------
// The general layer

static int validate_layer(const mta_layer_config *c, const mta_layer_weights *w)
{
    if (!c || !w) return MTA_ERR_NULL_ARG;
    if (c->batch < 0 || c->heads < 1 || c->seq_len < 0 || c->head_dim < 1 || c->c_h < 1 ||
        c->heads % c->c_h != 0)
        return MTA_ERR_BAD_SHAPE;
    const bool pre = w->kq_pre || w->conv3d;
    if (pre && (c->c_q < 1 || c->c_k < 1)) return MTA_ERR_BAD_SHAPE;
    if (w->kq_post && (c->c_q2 < 1 || c->c_k2 < 1)) return MTA_ERR_BAD_SHAPE;
    if (w->conv3d && (w->kq_pre || w->head_pre)) return MTA_ERR_BAD_PLACEMENT;
    if (c->exact != 0 && c->exact != 1) return MTA_ERR_BAD_PLACEMENT;
    if (c->dtype != MTA_F32 && c->dtype != MTA_BF16) return MTA_ERR_BAD_DTYPE;
    if (!(c->gn_eps > 0.0f) || !isfinite(c->gn_eps) || !isfinite(c->depth_scale)) return MTA_ERR_BAD_VALUE;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return MTA_ERR_UNSUPPORTED;
    if (c->c_h != 1 && c->c_h != 2 && c->c_h != 4) return MTA_ERR_UNSUPPORTED;
    if (pre && (c->c_q > mta::MAX_CQ || c->c_k > mta::MAX_CK)) return MTA_ERR_UNSUPPORTED;
    if (w->kq_post && (c->c_q2 > mta::MAX_CQ || c->c_k2 > mta::MAX_CK)) return MTA_ERR_UNSUPPORTED;
    if (c->seq_len > (1 << 24)) return MTA_ERR_UNSUPPORTED;
    const int64_t n_qt = (c->seq_len + mta::BM - 1) / mta::BM;
    if (n_qt * (int64_t)c->batch * (c->heads / c->c_h) > INT32_MAX) return MTA_ERR_UNSUPPORTED;
    return MTA_OK;
}

// A layer with exactly one key-query and one head convolution in one of
// mta_forward's placements (the key-query convolution first when both follow
// the softmax) is that placement.
static bool as_placement(const mta_layer_config *c, const mta_layer_weights *w, mta_config &sc,
                         const float *&th_kq, const float *&th_head)
{
    if (w->conv3d) return false;
    const int nkq = (w->kq_pre != nullptr) + (w->kq_post != nullptr);
    const int nh = (w->head_pre != nullptr) + (w->head_post != nullptr) + (w->head_post2 != nullptr);
    if (nkq != 1 || nh != 1) return false;
    if (w->kq_pre) {
        sc.kq_place = c->exact ? MTA_PRE_SOFTMAX_EXACT : MTA_PRE_SOFTMAX;
        sc.c_q = c->c_q;
        sc.c_k = c->c_k;
        th_kq = w->kq_pre;
    } else {
        if (w->head_post) return false;  // a head mix before the post-softmax convolution
        sc.kq_place = MTA_POST_SOFTMAX;
        sc.c_q = c->c_q2;
        sc.c_k = c->c_k2;
        th_kq = w->kq_post;
    }
    if (w->head_pre) {
        sc.head_place = MTA_PRE_SOFTMAX;
        th_head = w->head_pre;
    } else {
        sc.head_place = MTA_POST_SOFTMAX;
        th_head = w->head_post ? w->head_post : w->head_post2;
    }
    sc.batch = c->batch;
    sc.heads = c->heads;
    sc.seq_len = c->seq_len;
    sc.head_dim = c->head_dim;
    sc.c_h = c->c_h;
    sc.dtype = c->dtype;
    sc.gn_eps = c->gn_eps;
    sc.depth_scale = c->depth_scale;
    return true;
}

struct LayerPlan {
    mta::layer::LayerFn fn = nullptr;
    size_t lds = 0;
    int grid = 0;
    mta::layer::LParams p{};
};

static int make_layer_plan(const mta_layer_config *c, const mta_layer_weights *w, LayerPlan &pl)
{
    mta::layer::LParams &p = pl.p;
    const int ch = c->c_h, d = c->head_dim;
    p.H = c->heads;
    p.T = c->seq_len;
    p.G = c->heads / ch;
    p.units = c->batch * p.G;
    p.n_qt = (c->seq_len + mta::BM - 1) / mta::BM;
    p.pre = w->conv3d ? 2 : (w->kq_pre ? 1 : 0);
    p.exact = p.pre ? c->exact : 0;
    p.cq1 = p.pre ? c->c_q : 1;
    p.ck1 = p.pre ? c->c_k : 1;
    p.cq2 = w->kq_post ? c->c_q2 : 1;
    p.ck2 = w->kq_post ? c->c_k2 : 1;
    p.h2 = w->kq_post ? p.cq2 - 1 : 0;
    p.l2 = w->kq_post ? (p.ck2 + 1) / 2 - 1 : 0;
    const int r2 = w->kq_post ? p.ck2 / 2 : 0;
    p.h1 = p.pre ? p.cq1 - 1 : 0;
    p.l1 = p.pre ? (p.ck1 + 1) / 2 - 1 : 0;
    p.nLr = mta::BM + p.h2;
    p.nLc = mta::BN + p.l2 + r2;
    const int nlcb = (p.nLc + 15) / 16;
    p.lpitch = nlcb * 16 + 4;
    p.nSrb = p.pre ? (p.nLr + p.h1 + 15) / 16 : 0;
    p.nScb = p.pre ? (16 * nlcb + p.ck1 - 1 + 15) / 16 : 0;
    p.spitch = p.pre ? p.nScb * 16 + 4 : 0;
    p.ck1p = (p.ck1 + 3) & ~3;
    p.ck2p = (p.ck2 + 3) & ~3;
    p.sc = 1.4426950408889634f / sqrtf((float)d);
    p.eps = c->gn_eps;
    p.depth_scale = c->depth_scale;
    pl.grid = p.n_qt * p.units;
    const int kq1 = p.pre ? p.cq1 : 0, kk1 = p.pre ? p.ck1 : 0;
    const int kq2 = w->kq_post ? p.cq2 : 0, kk2 = w->kq_post ? p.ck2 : 0;
    if (c->dtype == MTA_BF16) {
        pl.fn = mta::find_launch_layer_bf16(d, ch, kq1, kk1, kq2, kk2);
        pl.lds = d == 32 ? mta::layer::llayout<mta::bf16_t, 32>(p, ch).total
                 : d == 64 ? mta::layer::llayout<mta::bf16_t, 64>(p, ch).total
                           : mta::layer::llayout<mta::bf16_t, 128>(p, ch).total;
    } else {
        pl.fn = mta::find_launch_layer_f32(d, ch, kq1, kk1, kq2, kk2);
        pl.lds = d == 32 ? mta::layer::llayout<float, 32>(p, ch).total
                 : d == 64 ? mta::layer::llayout<float, 64>(p, ch).total
                           : mta::layer::llayout<float, 128>(p, ch).total;
    }
    if (!pl.fn || pl.lds > 160 * 1024) return MTA_ERR_UNSUPPORTED;
    return MTA_OK;
}

// A layer whose only convolution is the both-pre-softmax 3D kernel (two-pass
// masks) runs the head-split kernel's 3D form where it is instantiated (bf16,
// d = 128, c_h = 2): the geometry of the default placement's plan, the 3D
// kernel in place of the per-head one and no head mix.
static bool as_v4_3d(const mta_layer_config *c, const mta_layer_weights *w, Plan &pl)
{
    if (!w->conv3d || w->kq_pre || w->head_pre || w->head_post || w->kq_post || w->head_post2) return false;
    if (c->dtype != MTA_BF16 || c->exact) return false;
    const mta::LaunchFn fn = mta::find_launch_v4_3d(c->head_dim, c->c_h, c->c_q, c->c_k);
    if (!fn) return false;
    mta_config sc{};
    sc.batch = c->batch; sc.heads = c->heads; sc.seq_len = c->seq_len; sc.head_dim = c->head_dim;
    sc.c_q = c->c_q; sc.c_k = c->c_k; sc.c_h = c->c_h;
    sc.kq_place = MTA_PRE_SOFTMAX; sc.head_place = MTA_POST_SOFTMAX;
    sc.dtype = c->dtype; sc.gn_eps = c->gn_eps; sc.depth_scale = c->depth_scale;
    if (validate(&sc) != MTA_OK || make_plan(&sc, pl) != MTA_OK) return false;
    if (!pl.name || std::strncmp(pl.name, "mta_fwd_v4", 10) != 0) return false;
    const size_t lds = (size_t)mta::v4::layout(c->c_q, c->c_k, false, false, true).total;
    if (lds > 160 * 1024) return false;
    pl.fn = fn;
    pl.lds = lds;
    pl.name = "mta_fwd_v4 (one pass, head-split waves, 3D convolution, fp16 matrix-core stencil)";
    return true;
}

// The repeated convolution (a key-query convolution before the softmax with
// the two-pass masks, and one after it; head mixes after the softmax or none)
// runs the head-split two-pass kernel where it is instantiated (bf16, d = 128,
// c_h = 2): the post-softmax stages fold into one 3D stencil.
struct RepPlan {
    mta::rep::RepFn fn = nullptr;
    size_t lds = 0;
    int grid = 0;
    mta::rep::RParams p{};
};

static const char *const REP_NAME =
    "mta_fwd_rep (two passes, head-split waves, the repeated convolution after the softmax as a 3D stencil, "
    "fp16 matrix-core stencils)";

static bool as_rep(const mta_layer_config *c, const mta_layer_weights *w, RepPlan &pl)
{
    if (!w->kq_pre || !w->kq_post || w->conv3d || w->head_pre || c->exact) return false;
    if (c->dtype != MTA_BF16 || c->head_dim != 128 || c->c_h != 2) return false;
    pl.fn = mta::rep::find_launch(c->head_dim, c->c_h, c->c_q, c->c_k, c->c_q2, c->c_k2);
    pl.lds = mta::rep::lds_bytes(c->c_q, c->c_k, c->c_q2, c->c_k2);
    if (!pl.fn || pl.lds == 0 || pl.lds > 160 * 1024) return false;
    mta::rep::RParams &p = pl.p;
    p.H = c->heads;
    p.T = c->seq_len;
    p.G = c->heads / 2;
    p.units = c->batch * p.G;
    p.n_qt = (c->seq_len + mta::BM - 1) / mta::BM;
    p.sc = 1.4426950408889634f / sqrtf((float)c->head_dim);
    p.eps = c->gn_eps;
    p.depth_scale = c->depth_scale;
    pl.grid = p.n_qt * p.units;
    return true;
}

int mta_forward_layer(const void *q, const void *k, const void *v, const mta_layer_weights *w,
                      const mta_layer_config *c, void *out, void *stream)
{
    const int vs = validate_layer(c, w);
    if (vs != MTA_OK) return vs;
    if (c->batch == 0 || c->seq_len == 0) return MTA_OK;
    mta_config sc;
    const float *th_kq = nullptr, *th_head = nullptr;
    if (as_placement(c, w, sc, th_kq, th_head))
        return forward_impl(q, k, v, th_kq, th_head, w->gn_w, w->gn_b, w->gate, &sc, out, stream);
    if (!q || !k || !v || !w->gn_w || !w->gn_b || !out) return MTA_ERR_NULL_ARG;
    const float *ws[] = {w->kq_pre, w->head_pre, w->conv3d, w->head_post, w->kq_post, w->head_post2,
                         w->gn_w, w->gn_b, w->gate};
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return MTA_ERR_MISALIGNED;
    for (const float *x : ws)
        if (x && !aligned4(x)) return MTA_ERR_MISALIGNED;
    Plan p3;
    if (as_v4_3d(c, w, p3)) {
        mta::Params &p = p3.p;
        p.q = q; p.k = k; p.v = v;
        p.theta = w->conv3d; p.wmix = nullptr; p.gn_w = w->gn_w; p.gn_b = w->gn_b; p.gate = w->gate;
        p.out = out;
        const hipError_t e = p3.fn(p, p3.grid, p3.lds, reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
    }
    RepPlan rp;
    if (as_rep(c, w, rp)) {
        mta::rep::RParams &p = rp.p;
        p.q = q; p.k = k; p.v = v;
        p.theta1 = w->kq_pre; p.w1 = w->head_post; p.theta2 = w->kq_post; p.w2 = w->head_post2;
        p.gn_w = w->gn_w; p.gn_b = w->gn_b; p.gate = w->gate;
        p.out = out;
        const hipError_t e = rp.fn(p, rp.grid, rp.lds, reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
    }
    LayerPlan pl;
    const int ps = make_layer_plan(c, w, pl);
    if (ps != MTA_OK) return ps;
    mta::layer::LParams &p = pl.p;
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.kq_pre = w->kq_pre; p.head_pre = w->head_pre; p.conv3d = w->conv3d;
    p.head_post = w->head_post; p.kq_post = w->kq_post; p.head_post2 = w->head_post2;
    p.gn_w = w->gn_w; p.gn_b = w->gn_b; p.gate = w->gate;
    const hipError_t e = pl.fn(p, pl.grid, pl.lds, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
}

const char *mta_layer_kernel_name(const mta_layer_config *c, const mta_layer_weights *w)
{
    if (validate_layer(c, w) != MTA_OK) return nullptr;
    mta_config sc;
    const float *th_kq = nullptr, *th_head = nullptr;
    if (as_placement(c, w, sc, th_kq, th_head)) return mta_kernel_name(&sc);
    Plan p3;
    if (as_v4_3d(c, w, p3)) return p3.name;
    RepPlan rp;
    if (as_rep(c, w, rp)) return REP_NAME;
    LayerPlan pl;
    return make_layer_plan(c, w, pl) == MTA_OK ? "mta_fwd_layer (general layer, two passes)" : nullptr;
}

// ---------------------------------------------------------------------------
// Backward

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The fused backward (mta_bwd.h): the default placement (key-query
// convolution before the softmax, head mix after it) with c_h <= 2, where its
// kernels are instantiated and fit in LDS.  Fills the shape fields of bp and
// the LDS sizes.
static bool fused_plan(const mta_config *cfg, mta::bwd::BParams &bp, size_t &lds_a, size_t &lds_b,
                       mta::bwd::BwdFn &fn);

static bool use_fused(const mta_config *cfg)
{
    mta::bwd::BParams bp{};
    size_t la, lb;
    mta::bwd::BwdFn fn;
    return fused_plan(cfg, bp, la, lb, fn);
}

size_t mta_backward_workspace_size(const mta_config *cfg)
{
    if (validate(cfg) != MTA_OK) return 0;
    if (!use_fused(cfg)) {
        if (cfg->seq_len > mta::gen::MAX_T) return 0;
        if (cfg->batch == 0 || cfg->seq_len == 0) return 0;
        return mta::gen::workspace_bytes(cfg->batch, cfg->heads, cfg->seq_len, cfg->head_dim, cfg->c_h,
                                         cfg->kq_place, cfg->head_place);
    }
    const size_t rows = (size_t)cfg->batch * cfg->heads * cfg->seq_len;
    // bf16: dO as high and low bf16 planes; fp32: one fp32 array
    const size_t planes = cfg->dtype == MTA_BF16 ? 2 : 1;
    const size_t el = cfg->dtype == MTA_BF16 ? 2 : 4;
    return 3 * align256(rows * 4) + planes * align256(rows * cfg->head_dim * el);
}

const char *mta_backward_kernel_name(const mta_config *cfg)
{
    if (validate(cfg) != MTA_OK) return nullptr;
    if (use_fused(cfg)) {
        const int bf = cfg->dtype == MTA_BF16;
        const bool prep = bf && cfg->head_dim == 128 && cfg->c_h == 2 &&
                          mta::find_launch_v4_prep(cfg->head_dim, cfg->c_h, cfg->c_q, cfg->c_k,
                                                   cfg->kq_place == MTA_PRE_SOFTMAX_EXACT) &&
                          mta::v4::layout(cfg->c_q, cfg->c_k, true).total <= 160 * 1024;
        return prep ? "mta_bwd (fused: head-split forward with the gradient epilogue + mta_bwd_main)"
                    : "mta_bwd (fused: mta_bwd_prep + mta_bwd_main)";
    }
    if (cfg->seq_len > mta::gen::MAX_T) return nullptr;
    return "mta_bwd_gen (per-head maps in the workspace)";
}

// The least workspace a call accepts: the fused backward needs
// mta_backward_workspace_size; the general one one head group's maps (it
// then processes the groups in more chunks).
static size_t workspace_min(const mta_config *cfg)
{
    if (use_fused(cfg)) return mta_backward_workspace_size(cfg);
    return mta::gen::unit_bytes(cfg->seq_len, cfg->head_dim, cfg->c_h, cfg->kq_place, cfg->head_place);
}

static int backward_impl(const void *q, const void *k, const void *v, const float *theta_kq,
                         const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                         const void *dout, const mta_config *cfg, float *dq, float *dk, float *dv,
                         float *dtheta_kq, float *dtheta_head, float *dgn_w, float *dgn_b, float *dgate,
                         void *workspace, size_t workspace_bytes, void *stream);

int mta_backward(const void *q, const void *k, const void *v, const float *theta_kq, const float *theta_head,
                 const float *gn_w, const float *gn_b, const float *gate, const void *dout,
                 const mta_config *cfg, float *dq, float *dk, float *dv, float *dtheta_kq, float *dtheta_head,
                 float *dgn_w, float *dgn_b, float *dgate, void *workspace, size_t workspace_bytes, void *stream)
{
    return backward_impl(q, k, v, theta_kq, theta_head, gn_w, gn_b, gate, dout, cfg, dq, dk, dv, dtheta_kq,
                         dtheta_head, dgn_w, dgn_b, dgate, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The backward without a caller workspace: the workspace is a file-scope device
// array, one per GPU the library runs on, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address): its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current.

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)72 << 20;
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES] = {};

// The scratch array's device address on the current device (NULL on failure).
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t mta_backward_scratch_bytes(void) { return SCRATCH_BYTES; }

int mta_backward_noalloc(const void *q, const void *k, const void *v, const float *theta_kq,
                         const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                         const void *dout, const mta_config *cfg, float *dq, float *dk, float *dv,
                         float *dtheta_kq, float *dtheta_head, float *dgn_w, float *dgn_b, float *dgate,
                         void *stream)
{
    const int vs = validate(cfg);
    if (vs != MTA_OK) return vs;
    if (cfg->batch == 0 || cfg->seq_len == 0) return MTA_OK;
    if (!use_fused(cfg) && cfg->seq_len > mta::gen::MAX_T) return MTA_ERR_UNSUPPORTED;
    if (workspace_min(cfg) > SCRATCH_BYTES) return MTA_ERR_SCRATCH;
    void *ws = scratch_on_current_device();
    if (!ws) return MTA_ERR_LAUNCH;
    return backward_impl(q, k, v, theta_kq, theta_head, gn_w, gn_b, gate, dout, cfg, dq, dk, dv, dtheta_kq,
                         dtheta_head, dgn_w, dgn_b, dgate, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"

extern "C" {

static bool fused_plan(const mta_config *cfg, mta::bwd::BParams &bp, size_t &lds_a, size_t &lds_b,
                       mta::bwd::BwdFn &fn)
{
    if (cfg->kq_place == MTA_POST_SOFTMAX || cfg->head_place != MTA_POST_SOFTMAX || cfg->c_h > 2) return false;
    const int d = cfg->head_dim, ch = cfg->c_h, cq = cfg->c_q, ck = cfg->c_k;
    const int bf = cfg->dtype == MTA_BF16;
    fn = mta::find_launch_bwd(bf, d, ch, cq, ck, cfg->kq_place == MTA_PRE_SOFTMAX_EXACT);
    if (!fn) return false;
    mta::Params &p = bp.f;
    p.H = cfg->heads; p.T = cfg->seq_len; p.c_q = cq; p.c_k = ck;
    p.G = cfg->heads / ch;
    p.units = cfg->batch * p.G;
    p.n_qt = (cfg->seq_len + mta::BM - 1) / mta::BM;
    p.head_pre = 0;
    p.exact = cfg->kq_place == MTA_PRE_SOFTMAX_EXACT;
    p.hl = (ck + 1) / 2 - 1;
    p.ncb = (mta::BN + ck - 1 + 15) / 16;
    p.pitch = p.ncb * 16 + 4;
    p.nbuf = 1;
    p.sc = 1.4426950408889634f / sqrtf((float)d);
    p.eps = cfg->gn_eps;
    p.depth_scale = cfg->depth_scale;
    bp.hr = ck / 2;
    bp.nEr = mta::BM + cq - 1;
    bp.nEc = mta::BN + ck - 1;
    const int nlcb = (bp.nEc + 15) / 16;
    bp.epitch = nlcb * 16 + 4;
    bp.nRrb = (bp.nEr + cq - 1 + 15) / 16;
    bp.nRcb = (16 * nlcb + ck - 1 + 15) / 16;
    bp.xpitch = bp.nRcb * 16 + 4;
    bp.inv_sqrt_d = 1.0f / sqrtf((float)d);
    bp.inv_log2e = 0.6931471805599453f;
    auto pad4 = [](size_t x) { return (x + 3) & ~(size_t)3; };
    const size_t ckp = (size_t)((ck + 3) & ~3);
    const size_t vb = bf ? (d == 32 ? mta::vbuf_bytes<mta::bf16_t, 32>()
                                    : d == 64 ? mta::vbuf_bytes<mta::bf16_t, 64>()
                                              : mta::vbuf_bytes<mta::bf16_t, 128>())
                         : (d == 32 ? mta::vbuf_bytes<float, 32>()
                                    : d == 64 ? mta::vbuf_bytes<float, 64>() : mta::vbuf_bytes<float, 128>());
    lds_a = ((size_t)mta::EXT_R * p.pitch + pad4(ch * cq * ckp) + pad4((size_t)ch * ch) +
                          (size_t)4 * ch * 2 * d + pad4((size_t)4 * ch)) * 4 + vb;
    const size_t nEr4 = pad4(bp.nEr);
    lds_b = ((size_t)bp.nRrb * 16 * bp.xpitch + (size_t)bp.nEr * bp.epitch +
                          (size_t)ch * bp.nEr * bp.epitch + pad4(ch * cq * ckp) + pad4((size_t)ch * ch) +
                          pad4(ch * cq * ckp) + (size_t)ch * 3 * nEr4 + pad4((size_t)mta::bwd::NWB * ch * ch)) * 4 + vb +
                          mta::bwd::ms_bytes(mta::bwd_fixed_sizes(bf, d, ch, cq, ck), bp.nRrb, ch, cq);
    return lds_a <= 160 * 1024 && lds_b <= 160 * 1024;
}

static int backward_impl(const void *q, const void *k, const void *v, const float *theta_kq,
                         const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                         const void *dout, const mta_config *cfg, float *dq, float *dk, float *dv,
                         float *dtheta_kq, float *dtheta_head, float *dgn_w, float *dgn_b, float *dgate,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    const int vs = validate(cfg);
    if (vs != MTA_OK) return vs;
    if (cfg->batch == 0 || cfg->seq_len == 0) return MTA_OK;
    if (!q || !k || !v || !theta_kq || !theta_head || !gn_w || !gn_b || !dout || !dq || !dk || !dv ||
        !dtheta_kq || !dtheta_head || !dgn_w || !dgn_b || !workspace || (gate && !dgate))
        return MTA_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return MTA_ERR_MISALIGNED;
    const float *fl[] = {theta_kq, theta_head, gn_w, gn_b, gate, dq, dk, dv, dtheta_kq, dtheta_head,
                         dgn_w, dgn_b, dgate};
    for (const float *x : fl)
        if (x && !aligned4(x)) return MTA_ERR_MISALIGNED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    mta::bwd::BParams bp{};
    size_t lds_a = 0, lds_b = 0;
    mta::bwd::BwdFn fn = nullptr;
    if (!fused_plan(cfg, bp, lds_a, lds_b, fn)) {
        // every other placement: the backward with the maps in the workspace
        if (cfg->seq_len > mta::gen::MAX_T) return MTA_ERR_UNSUPPORTED;
        if (workspace_bytes < workspace_min(cfg)) return MTA_ERR_BAD_VALUE;
        if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return MTA_ERR_MISALIGNED;
        mta::gen::GenArgs ga{};
        ga.q = q; ga.k = k; ga.v = v; ga.dout = dout;
        ga.theta = theta_kq; ga.w = theta_head; ga.gn_w = gn_w; ga.gn_b = gn_b; ga.gate = gate;
        ga.dq = dq; ga.dk = dk; ga.dv = dv; ga.dtheta = dtheta_kq; ga.dw = dtheta_head;
        ga.dgn_w = dgn_w; ga.dgn_b = dgn_b; ga.dgate = gate ? dgate : nullptr;
        ga.B = cfg->batch; ga.H = cfg->heads; ga.T = cfg->seq_len; ga.d = cfg->head_dim;
        ga.c_q = cfg->c_q; ga.c_k = cfg->c_k; ga.c_h = cfg->c_h;
        ga.kq_place = cfg->kq_place; ga.head_place = cfg->head_place; ga.bf16 = cfg->dtype == MTA_BF16;
        ga.eps = cfg->gn_eps; ga.depth_scale = cfg->depth_scale;
        return mta::gen::backward(ga, workspace, workspace_bytes, s) == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
    }
    if (workspace_bytes < mta_backward_workspace_size(cfg)) return MTA_ERR_BAD_VALUE;

    const int d = cfg->head_dim, ch = cfg->c_h, cq = cfg->c_q, ck = cfg->c_k;
    const int bf = cfg->dtype == MTA_BF16;
    mta::Params &p = bp.f;
    p.q = q; p.k = k; p.v = v;
    p.theta = theta_kq; p.wmix = theta_head; p.gn_w = gn_w; p.gn_b = gn_b; p.gate = gate;
    p.out = nullptr;
    bp.dout = dout;
    bp.dq = dq; bp.dk = dk; bp.dv = dv;
    bp.dtheta = dtheta_kq; bp.dw = dtheta_head; bp.dgn_w = dgn_w; bp.dgn_b = dgn_b; bp.dgate = dgate;
    const size_t rows = (size_t)cfg->batch * cfg->heads * cfg->seq_len;
    char *ws = static_cast<char *>(workspace);
    bp.ws_m = reinterpret_cast<float *>(ws);
    bp.ws_il = reinterpret_cast<float *>(ws + align256(rows * 4));
    bp.ws_D = reinterpret_cast<float *>(ws + 2 * align256(rows * 4));
    bp.ws_dO = ws + 3 * align256(rows * 4);
    bp.ws_dOl = ws + 3 * align256(rows * 4) + align256(rows * d * (bf ? 2 : 4));

    // bf16, d = 128, c_h = 2: the first kernel's work (row statistics, dO, D,
    // GroupNorm and gate gradients) is done by the one-pass head-split forward
    // with that epilogue, where it is instantiated and fits
    mta::PrepFn pfn = nullptr;
    size_t lds_v4 = 0;
    if (bf && d == 128 && ch == 2) {
        pfn = mta::find_launch_v4_prep(d, ch, cq, ck, p.exact);
        lds_v4 = (size_t)mta::v4::layout(cq, ck, true).total;
        if (lds_v4 > 160 * 1024) pfn = nullptr;
    }

    mta::bwd::ZeroList z{};
    z.p[0] = dq;          z.n[0] = rows * d;
    z.p[1] = dtheta_kq;   z.n[1] = (size_t)cfg->heads * cq * ck;
    z.p[2] = dtheta_head; z.n[2] = (size_t)p.G * ch * ch;
    z.p[3] = dgn_w;       z.n[3] = (size_t)cfg->heads * d;
    z.p[4] = dgn_b;       z.n[4] = (size_t)cfg->heads * d;
    z.k = 5;
    if (dgate) {
        z.p[5] = dgate;
        z.n[5] = (size_t)cfg->heads;
        z.k = 6;
    }
    hipError_t e = mta::launch_fill_zero(z, s);
    if (e != hipSuccess) return MTA_ERR_LAUNCH;
    const int grid = p.n_qt * p.units;
    if (pfn) {
        mta::Params pv = p;
        pv.ncb = 5;
        pv.pitch = pv.ncb * 16 + 4;
        mta::v4::PrepArgs pa{static_cast<const mta::bf16_t *>(dout), bp.ws_m, bp.ws_il, bp.ws_D,
                             static_cast<mta::bf16_t *>(bp.ws_dO), static_cast<mta::bf16_t *>(bp.ws_dOl),
                             dgn_w, dgn_b, dgate};
        e = pfn(pv, pa, grid, lds_v4, s);
        if (e != hipSuccess) return MTA_ERR_LAUNCH;
        e = fn(bp, 0, lds_a, grid, lds_b, s);  // the main kernel only
    } else {
        e = fn(bp, grid, lds_a, grid, lds_b, s);
    }
    return e == hipSuccess ? MTA_OK : MTA_ERR_LAUNCH;
}

}  // extern "C"
