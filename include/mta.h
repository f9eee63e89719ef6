/*
 * mta.h — C ABI of the MI355X (gfx950) Multi-Token Attention forward.
 *
 * The operation is the MTA attention forward of the page "Multi-Token
 * Attention — Paper Graph" (summary of arXiv 2504.00927), section 3.4:
 *   1. logits  Ahat = Q K^T / sqrt(d)               ("Standard Multi-Head
 *      Attention");
 *   2. key-query convolution Conv2d_theta over the (query, key) plane of each
 *      head, kernel c_q x c_k, either before the softmax with two-pass masking
 *      Softmax(Mask_-inf(Conv2d(Mask_0(Ahat)))), or before it in the exact
 *      form of Eq. 4, whose indicator 1{i >= j-j'} keeps a tap iff its key is
 *      not in the future of the output query i (the unmasked logits are
 *      convolved, then Mask_-inf), or after it,
 *      Mask_0(Conv2d(Softmax(Mask_-inf(Ahat))))     ("Key-Query Convolution",
 *      Eq. 4 and the two-pass / post-softmax forms);
 *   3. head mixing within non-overlapping groups of c_h heads,
 *      A^a_new = sum_b w_ab A^b, after the softmax (Eq. 7) or on the logits
 *      before it                                    ("Head Mixing Convolution");
 *   4. O^h = A^h V^h per head;
 *   5. GroupNorm over each head's d channels with a per-channel affine, times
 *      a scalar depth scale                         ("Group Normalization with
 *      Sigmoid Gating" / the overview page's "Group Normalization with Depth
 *      Scaling").
 * When both convolutions sit on the same side of the softmax the key-query
 * convolution runs first.  Positions outside [0, T) are zero padding for the
 * key-query convolution.  The scale is fixed at 1/sqrt(d).
 *
 * Conventions
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous,
 *    16-byte aligned.  The library allocates no memory and keeps no state
 *    between calls; calls are thread-safe.
 *  - The call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  The caller keeps every buffer alive until the stream work is
 *    done.  `cfg` is read before the call returns.
 *  - Errors: validation runs on the host before any device work.  On a
 *    negative return nothing was launched and `out` is untouched.  A device
 *    fault surfaces at the caller's next synchronisation.  No exception
 *    crosses the ABI and the library prints nothing.
 */
#ifndef MTA_H_
#define MTA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Placement of a convolution relative to the softmax.  MTA_PRE_SOFTMAX_EXACT
 * is valid for kq_place only: the key-query convolution before the softmax
 * with Eq. 4's exact causal indicator instead of the two-pass masks. */
#define MTA_PRE_SOFTMAX 0
#define MTA_POST_SOFTMAX 1
#define MTA_PRE_SOFTMAX_EXACT 2

/* Element type of q, k, v and out.  Kernels and GroupNorm parameters are
 * always float32.  Intermediate arithmetic is float32 (contractions accumulate
 * in float32 on the matrix cores; with MTA_BF16 the probabilities enter the A·V
 * product as bf16), with one exception: for MTA_BF16 the key-query convolution
 * of the head-split kernels runs on the matrix cores with fp16 operands (the logits or probabilities and the taps rounded to nearest,
 * 11 significant bits; magnitudes beyond 65504 clamped to 65504, which only
 * logits past ~5800 in natural units reach) and float32 accumulation.  Before
 * the softmax the centre tap (query offset 0, key offset 0) keeps float32
 * accuracy: the head-split kernels apply it to the float32 logits, so a
 * kernel near the identity stays accurate at large logits.  The head-split kernels (bf16, d = 128, head mix after the softmax,
 * the instantiated kernel sizes, c_h 1, 2 or 4) round each head's
 * probabilities to bf16 before the head mix, which they apply to the per-head
 * A·V products: under strongly cancelling mixing weights the output's error
 * relative to its size grows accordingly.  With groups of 8 or 16 heads they
 * run A·V with fp16 operands instead (11 significant bits: the probabilities,
 * and V converted exactly for 2^-14 <= |v| <= 65504, magnitudes beyond 65504
 * clamped, smaller ones rounded to the fp16 subnormal grid), which keeps that
 * growth within the bf16 tolerance.  Groups of 4 or more heads sum the
 * source head pairs' shares in float32.
 * mta_kernel_name tells which kernel a configuration runs. */
#define MTA_F32 0
#define MTA_BF16 1

/* Status codes. */
#define MTA_OK 0
#define MTA_ERR_NULL_ARG -1      /* a required pointer is NULL                 */
#define MTA_ERR_BAD_SHAPE -2     /* B,H,T < 0, H % c_h != 0, kernel size < 1   */
#define MTA_ERR_BAD_PLACEMENT -3 /* kq_place not 0..2 or head_place not 0..1  */
#define MTA_ERR_BAD_DTYPE -4     /* dtype not MTA_F32 / MTA_BF16               */
#define MTA_ERR_MISALIGNED -5    /* a tensor pointer is not 16-byte aligned    */
#define MTA_ERR_UNSUPPORTED -6   /* valid but outside the library's limits:
                                    head_dim not in {32,64,128}, c_h not in
                                    {1,2,4,8,16} (8, 16: see mta_config),
                                    c_q > 16, c_k > 31, T > 2^24, or no kernel
                                    of the configuration fits the LDS       */
#define MTA_ERR_LAUNCH -7        /* the kernel launch reported an error        */
#define MTA_ERR_BAD_VALUE -8     /* gn_eps <= 0 or not finite, depth_scale not
                                    finite                                      */
#define MTA_ERR_SCRATCH -9       /* mta_backward_noalloc: the problem needs more
                                    workspace than the device scratch array
                                    holds (mta_backward_scratch_bytes)          */

/* Problem description (all fields read synchronously). */
typedef struct mta_config {
    int32_t batch;      /* B >= 0                                              */
    int32_t heads;      /* H >= 1, a multiple of c_h                           */
    int32_t seq_len;    /* T >= 0                                              */
    int32_t head_dim;   /* d in {32, 64, 128}                                  */
    int32_t c_q;        /* key-query kernel size along queries, 1..16         */
    int32_t c_k;        /* key-query kernel size along keys, 1..31            */
    int32_t c_h;        /* heads per mixing group, 1, 2, 4, 8 or 16 (8 and 16: */
                        /* the forward only with MTA_BF16, d = 128, head mix  */
                        /* after the softmax, c_q x c_k 1x1, 4x9, 6x11, 8x15) */
    int32_t kq_place;   /* MTA_PRE_SOFTMAX (two-pass masking) | MTA_POST_SOFTMAX
                           | MTA_PRE_SOFTMAX_EXACT (Eq. 4's indicator)     */
    int32_t head_place; /* MTA_PRE_SOFTMAX | MTA_POST_SOFTMAX                  */
    int32_t dtype;      /* MTA_F32 | MTA_BF16                                  */
    float gn_eps;       /* GroupNorm epsilon (> 0), e.g. 1e-5                  */
    float depth_scale;  /* scalar applied after the affine, e.g. 1/sqrt(layer) */
} mta_config;

/*
 * mta_forward — the whole MTA attention forward (steps 1-5 above).
 *
 *  q, k, v     [B][H][T][d] of cfg->dtype, row-major.
 *  theta_kq    float32 [H][c_q][c_k]; element [h][i'][jj] weighs query offset
 *              i' (0 = the current query, i' > 0 = earlier queries) and key
 *              offset j' = jj - floor(c_k/2), which reads key j - j'
 *              (j' runs over [-floor(c_k/2), ceil(c_k/2)-1]).  The identity
 *              kernel is 1 at [h][0][floor(c_k/2)].
 *  theta_head  float32 [H/c_h][c_h][c_h]; element [g][a][b] is the weight of
 *              source head g*c_h+b in output head g*c_h+a (heads are grouped
 *              contiguously).
 *  gn_w, gn_b  float32 [H][d]: GroupNorm affine per head and channel.
 *  cfg         problem description.
 *  out         [B][H][T][d] of cfg->dtype; every element is written.
 *  stream      hipStream_t to launch on (NULL: default stream).
 * Returns MTA_OK or a negative MTA_ERR_* code (see above).  B == 0 or T == 0
 * returns MTA_OK without launching.
 */
int mta_forward(const void *q, const void *k, const void *v,
                const float *theta_kq, const float *theta_head,
                const float *gn_w, const float *gn_b,
                const mta_config *cfg, void *out, void *stream);

/*
 * mta_forward_gated — the same forward with the sigmoid-gated GroupNorm of
 * "Group Normalization with Sigmoid Gating" (page "Multi-Token Attention —
 * Paper Graph", section 3.4): each head's normalised, affine-transformed output
 * is multiplied by sigmoid(gate[h]) (and by cfg->depth_scale; pass 1 for the
 * gate alone).
 *
 *  gate        float32 [H] device pointer: one gate logit per head (not NULL;
 *              MTA_ERR_NULL_ARG otherwise; 4-byte aligned).
 *  Every other argument and every error code as for mta_forward.
 */
int mta_forward_gated(const void *q, const void *k, const void *v,
                      const float *theta_kq, const float *theta_head,
                      const float *gn_w, const float *gn_b, const float *gate,
                      const mta_config *cfg, void *out, void *stream);

/*
 * The general MTA layer: every stage of "Putting Everything Together" (page
 * "Multi-Token Attention — Paper Graph", section 3.4), each optional (NULL =
 * absent), in this order:
 *   L = S,  or Conv2d_kq_pre(Mask_0(S)) (Eq. 4's indicator when `exact`),  or
 *       the both-pre-softmax 3D convolution L^a = sum_b Conv2d_conv3d[a][b](.)
 *   L = head mix head_pre (L)                  (not with conv3d)
 *   P = softmax(Mask_-inf(L))
 *   P = head mix head_post (P)                 (Eq. 7)
 *   P = Mask_0(Conv2d_kq_post(P))              (key-query convolution after it)
 *   P = head mix head_post2 (P)                (the repeated head convolution)
 *   O^h = P^h V^h;  GroupNorm over d, times depth_scale (and sigmoid(gate[h])).
 * The repeated MTA convolution of the overall flow is kq_pre + head_post +
 * kq_post + head_post2.  A head mix maps source head b to output head a of a
 * group as in mta_forward; the key-query kernels use mta_forward's layout.
 */
typedef struct {
    const float *kq_pre;     /* [H][c_q][c_k] or NULL                              */
    const float *head_pre;   /* [H/c_h][c_h][c_h] or NULL                          */
    const float *conv3d;     /* [H/c_h][c_h][c_h][c_q][c_k] ([g][a][b]) or NULL;    */
                             /* excludes kq_pre and head_pre                        */
    const float *head_post;  /* [H/c_h][c_h][c_h] or NULL                          */
    const float *kq_post;    /* [H][c_q2][c_k2] or NULL                            */
    const float *head_post2; /* [H/c_h][c_h][c_h] or NULL                          */
    const float *gn_w, *gn_b;/* [H][d], required                                   */
    const float *gate;       /* [H] gate logits or NULL                            */
} mta_layer_weights;

typedef struct {
    int32_t batch, heads, seq_len, head_dim;
    int32_t c_q, c_k;        /* kernel size of kq_pre / conv3d (ignored without)   */
    int32_t c_q2, c_k2;      /* kernel size of kq_post (ignored without)           */
    int32_t c_h;
    int32_t exact;           /* 1: the pre-softmax convolution uses Eq. 4's         */
                             /* indicator instead of the two-pass Mask_0            */
    int32_t dtype;           /* MTA_F32 | MTA_BF16                                 */
    float gn_eps, depth_scale;
} mta_layer_config;

/*
 * mta_forward_layer — the general layer.  Pointers, layouts, alignment,
 * asynchrony and error codes as for mta_forward; weights and cfg must be non
 * NULL, gn_w and gn_b are required; conv3d together with kq_pre or head_pre is
 * MTA_ERR_BAD_PLACEMENT.  A layer that is one of mta_forward's placements runs
 * mta_forward's kernels; a layer whose only convolution is conv3d (two-pass
 * masks) runs the head-split kernel's 3D form where it is built (bf16,
 * head_dim 128, c_h 2, 6x11 or 1x1); the repeated form (kq_pre with the
 * two-pass masks and kq_post, head_post and head_post2 each optional, no
 * head_pre) runs a head-split two-pass kernel where it is built (bf16,
 * head_dim 128, c_h 2, c_q x c_k and c_q2 x c_k2 both 6x11 or both 4x9;
 * fp16 operands in both convolutions as in mta_forward, the first one's
 * centre tap applied to the float32 logits); any other layer runs the general layer
 * kernel, limited to c_q, c_q2 <= 16, c_k, c_k2 <= 31 and 160 KB of LDS per
 * workgroup (MTA_ERR_UNSUPPORTED beyond).
 */
int mta_forward_layer(const void *q, const void *k, const void *v, const mta_layer_weights *weights,
                      const mta_layer_config *cfg, void *out, void *stream);

/* Host-only: the kernel mta_forward_layer launches for a layer, or NULL if the
 * layer is invalid or unsupported (weights' pointers are only tested for NULL). */
const char *mta_layer_kernel_name(const mta_layer_config *cfg, const mta_layer_weights *weights);

/*
 * mta_backward — gradients of mta_forward (mta_forward_gated when gate is not
 * NULL) for every placement of the two convolutions (kq_place, head_place),
 * c_h in {1, 2, 4, 8, 16}, d in {32, 64, 128}, either dtype: the chain rule of the
 * forward of page "Multi-Token Attention — Paper Graph", section 3.4 ("Key-Query
 * Convolution" Eq. 4 and its transpose, the softmax, "Head Mixing Convolution"
 * Eq. 7, A.V, "Group Normalization with Sigmoid Gating").  Given
 * dout = dL/dout [B][H][T][d] (input dtype) it writes, in float32:
 *   dq, dk, dv       [B][H][T][d]
 *   dtheta_kq        [H][c_q][c_k]
 *   dtheta_head      [H/c_h][c_h][c_h]
 *   dgn_w, dgn_b     [H][d]
 *   dgate            [H] (required if and only if gate is given)
 * Two implementations (mta_backward_kernel_name tells which one a
 * configuration runs):
 *   - the default placement (kq_place MTA_PRE_SOFTMAX or MTA_PRE_SOFTMAX_EXACT,
 *     head_place MTA_POST_SOFTMAX) with c_h <= 2 is fused per tile: nothing of
 *     size T x T is stored; the workspace holds row statistics and dO;
 *   - every other configuration keeps each head's T x T maps (float32, the
 *     causal band of 64 x 64 tiles) in the workspace and computes in float32
 *     throughout; T <= 32768 (MTA_ERR_UNSUPPORTED beyond).  Head groups are
 *     processed in as many chunks as the workspace needs.
 * `workspace` is a device buffer, 256-byte aligned, owned by the caller, of
 * mta_backward_workspace_size(cfg) bytes (the fused form needs exactly that;
 * the map form accepts less, down to one head group's maps, and then runs more
 * chunks); its contents are scratch (undefined after the call).  Too small a
 * workspace is MTA_ERR_BAD_VALUE.  Asynchronous on `stream`; every output is
 * overwritten.  Other arguments and error codes as mta_forward.
 */
int mta_backward(const void *q, const void *k, const void *v, const float *theta_kq, const float *theta_head,
                 const float *gn_w, const float *gn_b, const float *gate, const void *dout,
                 const mta_config *cfg, float *dq, float *dk, float *dv, float *dtheta_kq,
                 float *dtheta_head, float *dgn_w, float *dgn_b, float *dgate, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Bytes of workspace mta_backward asks for cfg: the fused form's need, or the
 * map form's maps for all head groups at once, capped at 16 GiB (at least one
 * head group).  0 if cfg is invalid or unsupported. */
size_t mta_backward_workspace_size(const mta_config *cfg);

/* Host-only: which backward mta_backward runs for cfg (a static string), or
 * NULL if cfg is invalid or unsupported. */
const char *mta_backward_kernel_name(const mta_config *cfg);

/*
 * mta_backward_noalloc — mta_backward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving or training loops,
 * harnesses that forbid hipMalloc): the same computation and arguments without
 * `workspace` / `workspace_bytes`.  Its workspace is a device array inside the
 * library, mta_backward_scratch_bytes() bytes (72 MiB: the 4K-context
 * workload's 65.5 MiB fits), one per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  A problem
 * whose least workspace exceeds the array (the fused form's
 * mta_backward_workspace_size, or one head group's maps) returns
 * MTA_ERR_SCRATCH before any device work.  Every call on a GPU uses that GPU's one array:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Nothing in the array needs clearing between
 * calls (the kernels write every workspace entry before reading it).
 */
int mta_backward_noalloc(const void *q, const void *k, const void *v, const float *theta_kq,
                         const float *theta_head, const float *gn_w, const float *gn_b, const float *gate,
                         const void *dout, const mta_config *cfg, float *dq, float *dk, float *dv,
                         float *dtheta_kq, float *dtheta_head, float *dgn_w, float *dgn_b, float *dgate,
                         void *stream);

/* Size in bytes of mta_backward_noalloc's device scratch array. */
size_t mta_backward_scratch_bytes(void);

/* Host-only: the name of the kernel mta_forward / mta_forward_gated launch for
 * this configuration (a static string, e.g. "mta_fwd_v4 (one pass,
 * head-split waves, fp16 matrix-core stencil)"), or NULL if the configuration is invalid or
 * unsupported.  For profiling and reports; it launches nothing. */
const char *mta_kernel_name(const mta_config *cfg);

/* Host-only check of a configuration against the library's limits: the same
 * validation and kernel selection (LDS fit included) that mta_forward runs,
 * pointer checks excepted.  Returns MTA_OK or the MTA_ERR_* code mta_forward
 * would return. */
int mta_check_config(const mta_config *cfg);

/* Static description of a status code (never NULL). */
const char *mta_status_string(int status);

/* ABI version: 100 * major + minor. */
int mta_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTA_H_ */
