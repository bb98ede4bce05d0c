/*
 * dp.h -- C ABI of the displaced-patch layer hot path on one MI355X (gfx950).
 *
 * Displaced patch parallelism (DistriFusion) splits a diffusion model's input
 * into patches, one per device, and lets every patch use the previous
 * denoising step's activations as context for the current one ("activation
 * displacement": "DistriFusion: Distributed Parallel Inference for
 * High-Resolution Diffusion Models", study.space page, Method; the abstract on
 * the scholarfeed.org author page).  This library computes one patch's share
 * of a UNet layer step on one GPU:
 *
 *   dp_groupnorm_async   corrected asynchronous GroupNorm (fresh local
 *                        statistics + stale statistics of the other patches)
 *   dp_conv3x3_halo      3x3 conv whose rows above/below the patch come from
 *                        the previous step's (stale) map (and a variant on
 *                        weights packed once by dp_conv3x3_pack_weights)
 *   dp_attention_splice  attention: queries from the fresh patch, keys and
 *                        values from the full stale map with the patch
 *                        spliced in
 *   dp_stale_update      writes the fresh patch into the resident stale map
 *   dp_linear            y = x W^T + b, the Q/K/V/O projections of an attention
 *                        layer whose K/V cache holds projected keys and values
 *   dp_conv3x3_halo_residual, dp_linear_residual
 *                        the conv and the projection with a block's skip
 *                        connection added before rounding
 *   dp_groupnorm_conv3x3_halo
 *                        GroupNorm (+SiLU) and the conv that consumes it in
 *                        one call, the normalisation folded into the conv
 *   dp_linear_qkv        the Q, K and V projections in one launch
 *
 * Geometry.  Maps are NHWC, batch-major: element (b, r, c, ch) of a [B][H][W][C]
 * map sits at ((b*H + r)*W + c)*C + ch.  The P patches are equal row bands:
 * patch i owns rows [i*h, (i+1)*h) with h = H/P (H must be divisible by P).
 * A patch buffer holds just its band, [B][h][W][C].  Token n of a map is row
 * n / W, column n % W, so a band is one contiguous token range per batch.
 *
 * Data types.  DP_F32: activations and weights are float.  DP_BF16:
 * activations and weights are bfloat16 (raw 16-bit patterns), arithmetic is
 * fp32 (MFMA accumulates in fp32), outputs are rounded to nearest even.
 * Statistics, bias, gamma and beta are always float.
 *
 * Ownership.  Every pointer argument except `p` and size outputs is device
 * memory owned by the caller (e.g. a torch tensor's storage).  The library
 * allocates nothing, keeps no state between calls and never synchronises the
 * host: each call only enqueues kernels on `stream` (0 = legacy default
 * stream) and returns.  Pointers must be 16-byte aligned.  A workspace `ws`
 * is caller-provided scratch of at least the size the matching *_ws query
 * returns (may be NULL when that size is 0); its contents on entry do not
 * matter and are undefined on return.  Calls that share a workspace or an
 * output must be ordered on one stream.
 *
 * Errors.  All arguments are validated on the host before anything is
 * enqueued; a rejected call enqueues nothing.  Return codes:
 *   DP_OK               enqueued
 *   DP_ERR_ARG          invalid argument (shape, index, NULL, alignment,
 *                       workspace too small, output overlapping an input)
 *   DP_ERR_UNSUPPORTED  valid but not built (e.g. bf16 attention with a
 *                       head_dim other than 64, or B > 65535: the batch
 *                       is a grid dimension of several kernels)
 *   DP_ERR_HIP          a HIP launch failed
 * dp_last_error() then describes the failure.  No C++ exception or abort
 * crosses the ABI.  Results are deterministic: repeated calls with the same
 * inputs give bitwise identical outputs (fixed reduction orders, no atomics
 * on data).
 */
#ifndef DP_H
#define DP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DP_OK = 0, DP_ERR_ARG = 1, DP_ERR_UNSUPPORTED = 2, DP_ERR_HIP = 3 } dp_status;

typedef enum { DP_F32 = 0, DP_BF16 = 1 } dp_dtype;

/* GroupNorm statistics a patch normalises with.  The three alternatives to
 * the corrected form are the ablations of the DistriFusion summary on
 * atlas.scime.ai, table "Measured effects reported in the paper"
 * (on-device patch statistics only; stale statistics reused).  The
 * synchronised exact form is DP_GN_CORRECTED with a table that holds the
 * current step's statistics of every band (warm-up). */
typedef enum {
    DP_GN_CORRECTED = 0, /* fresh moments of patch i + stale moments of the other bands */
    DP_GN_LOCAL = 1,     /* fresh moments of patch i only                              */
    DP_GN_STALE = 2      /* previous step's moments of all bands                       */
} dp_gn_mode;

typedef enum { DP_ACT_NONE = 0, DP_ACT_SILU = 1 } dp_act;

/* Full-map geometry and the patch this call computes: map [B][H][W][C],
 * P row bands, patch index i in [0, P). */
typedef struct {
    int32_t B, H, W, C, P, i;
} dp_patch;

/* ------------------------------------------------------------------------
 * dp_groupnorm_async -- corrected asynchronous GroupNorm of patch i.
 *
 * Source: DistriFusion summary (atlas.scime.ai), Approach: a corrected
 * asynchronous GroupNorm fixes the statistics that stale activations would
 * otherwise give; same page, "Measured effects" table: on-device-only and
 * stale-only statistics are the worse ablations, synchronised statistics the
 * slower exact one.  Reading: the patch normalises with the moments of the
 * spliced map (previous step's map with its own band fresh), per (b, group g):
 *   m_i, q_i   = mean of x and of x*x over the band's h*W*(C/G) elements
 *   CORRECTED: E = (m_i + sum_{j!=i} m'_j) / P,  Q = (q_i + sum_{j!=i} q'_j) / P
 *   LOCAL:     E = m_i,                          Q = q_i
 *   STALE:     E = sum_j m'_j / P,               Q = sum_j q'_j / P
 *   var = max(Q - E*E, 0),  y = (x - E) / sqrt(var + eps) * gamma[c] + beta[c]
 *   then y = y * sigmoid(y) if act == DP_ACT_SILU.
 *
 *   x_patch         [B][h][W][C] dtype, the fresh band
 *   stale_stats     [P][B][G][2] float, (m'_j, q'_j) of every band from the
 *                   previous step; may be NULL for DP_GN_LOCAL
 *   gamma, beta     [C] float or NULL (1 and 0)
 *   fresh_stats_out [B][G][2] float, receives (m_i, q_i); may be NULL; in
 *                   DP_GN_CORRECTED mode it may be slot i of stale_stats
 *                   (that mode never reads slot i), which splices the fresh
 *                   moments into the table without a separate copy
 *   y_patch         [B][h][W][C] dtype, or NULL to compute statistics only
 *                   (the first pass of a synchronous warm-up step); may equal
 *                   x_patch (in place) but must not otherwise overlap it
 *   ws              >= dp_groupnorm_async_ws bytes
 * Requires C % G == 0, C % 8 == 0 and C <= 8192 (bf16) or C % 4 == 0 and
 * C <= 4096 (f32), eps > 0; other channel counts give DP_ERR_UNSUPPORTED.
 * The normalising kernel's block holds one thread per group at least, so
 * G <= 1024; a G whose blocks would exceed 1024 threads or 64 KB of LDS is
 * rejected with DP_ERR_UNSUPPORTED before anything is enqueued.
 * After the call, fresh_stats_out is what dp_stale_update copies into slot i
 * of the table for the next step (see dp_stale_update).
 * ---------------------------------------------------------------------- */
dp_status dp_groupnorm_async_ws(const dp_patch* p, dp_dtype dtype, int32_t G, size_t* ws_bytes);

dp_status dp_groupnorm_async(const dp_patch* p, dp_dtype dtype, int32_t G, float eps,
                             dp_gn_mode mode, dp_act act, const void* x_patch,
                             const float* stale_stats, const float* gamma, const float* beta,
                             float* fresh_stats_out, void* y_patch, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_groupnorm_async_noalloc -- dp_groupnorm_async without a workspace, for
 * callers that cannot allocate device memory around the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, results and errors as dp_groupnorm_async (same kernels, bitwise
 * the same outputs), minus ws and ws_bytes: the statistics partials live in a
 * static device array of DP_NOALLOC_SCRATCH_BYTES bytes that every GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * and calls no allocating routine; its first call on a device looks up that
 * device's address of the array once.  A call whose partials need more than
 * DP_NOALLOC_SCRATCH_BYTES (B * nblk * G * 8 bytes, nblk <= 256 statistics
 * blocks per batch; dp_groupnorm_async_ws reports the size) gives
 * DP_ERR_UNSUPPORTED before anything is enqueued.  All calls on one GPU share
 * the array: calls that may run at the same time on one GPU (on different
 * streams, or from different threads without ordering) race and must not be
 * issued; calls ordered on one stream are safe.  The array needs no clearing:
 * each call writes every partial it reads.
 * ---------------------------------------------------------------------- */
#define DP_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

dp_status dp_groupnorm_async_noalloc(const dp_patch* p, dp_dtype dtype, int32_t G, float eps,
                                     dp_gn_mode mode, dp_act act, const void* x_patch,
                                     const float* stale_stats, const float* gamma, const float* beta,
                                     float* fresh_stats_out, void* y_patch, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_conv3x3_halo -- 3x3 convolution of patch i with stale halo rows.
 *
 * Source: study.space page, Method (previous-step activations give each
 * patch its context; each device computes only its patch).  Reading: the
 * conv is the zero-padded, stride-1 3x3 cross-correlation of the spliced
 * map, evaluated on the band's rows:
 *   y[b,y,x,o] = bias[o] + sum_{ky,kx,c} w[o,ky,kx,c] * src(b, r0+y+ky-1, x+kx-1, c)
 * where src is x_patch inside rows [r0, r0+h), x_stale at other rows of the
 * image (only rows r0-1 and r0+h are ever read) and 0 outside the image.
 *
 *   x_patch  [B][h][W][Cin] dtype (Cin = p->C)
 *   x_stale  [B][H][W][Cin] dtype, previous step's map
 *   w        [Cout][3][3][Cin] dtype
 *   bias     [Cout] float or NULL
 *   y_patch  [B][h][W][Cout] dtype; must not overlap any input
 *   ws       >= dp_conv3x3_halo_ws bytes
 * bf16 requires Cin % 64 == 0 and Cout % 32 == 0 (MFMA path), fewer than
 * 2^31 elements per batch image (H*W*Cin), fewer than 2^31 output pixels
 * (B*h*W) and weights under 2 GiB; f32 takes any Cin, Cout >= 1.
 * ---------------------------------------------------------------------- */
dp_status dp_conv3x3_halo_ws(const dp_patch* p, dp_dtype dtype, int32_t Cout, size_t* ws_bytes);

dp_status dp_conv3x3_halo(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                          const void* x_stale, const void* w, const float* bias, void* y_patch,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_conv3x3_pack_weights / dp_conv3x3_halo_packed -- the same convolution
 * with the weights in a packed layout the kernels read as whole cache lines.
 *
 * Source: as dp_conv3x3_halo (study.space page, Method); the layout is an
 * implementation detail of the bf16 kernels and does not change the result:
 * dp_conv3x3_halo_packed(w_packed) is bitwise equal to dp_conv3x3_halo(w).
 * Packed layout (bf16): element (co, ky, kx, ci) of w[Cout][3][3][Cin] at
 *   w_packed[ky][ci / 32][kx][co][ci % 32],
 * i.e. each (kernel row, 32-channel chunk) is one contiguous block of
 * 3 x Cout rows of 64 bytes.  Weights are constant across steps, so a layer
 * packs them once.
 *
 *   dp_conv3x3_packed_weights_bytes  bytes of w_packed (9*Cin*Cout*2), or 0
 *                                    when Cin or Cout < 1
 *   dp_conv3x3_pack_weights          w [Cout][3][3][Cin] bf16 -> w_packed
 *                                    (caller-owned, that many bytes, must not
 *                                    overlap w); enqueued on `stream`
 *   dp_conv3x3_halo_packed           arguments and errors as dp_conv3x3_halo,
 *                                    with w_packed in place of w
 * bf16 only (DP_ERR_UNSUPPORTED for DP_F32); Cin % 64 == 0, Cout % 32 == 0.
 * ---------------------------------------------------------------------- */
size_t dp_conv3x3_packed_weights_bytes(int32_t Cin, int32_t Cout);

dp_status dp_conv3x3_pack_weights(dp_dtype dtype, int32_t Cin, int32_t Cout, const void* w, void* w_packed,
                                  hipStream_t stream);

dp_status dp_conv3x3_halo_packed(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                                 const void* x_stale, const void* w_packed, const float* bias, void* y_patch,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_conv3x3_halo_residual -- the same convolution with a residual added:
 *   y[b,y,x,o] = (conv of dp_conv3x3_halo)[b,y,x,o] + residual[b,y,x,o]
 * with the sum formed in fp32 before the single rounding of the output.
 *
 * Source: the convolution as dp_conv3x3_halo (study.space page, Method).  The
 * residual is the skip connection of a UNet ResNet block (the denoiser of the
 * DistriFusion summary's experiments is SDXL, a U-Net; AsyncDiff rebuttal on
 * paperhub.cn, answer to Q2, speaks of the U-Net's blocks and their hidden
 * states): the block's second conv adds the block input of the same band.
 * The residual is fresh data of band i only, so displacement does not touch it.
 *
 *   w          [Cout][3][3][Cin] (w_packed == 0) or the packed layout of
 *              dp_conv3x3_pack_weights (w_packed == 1, bf16 only)
 *   residual   [B][h][W][Cout] dtype, or NULL (then exactly dp_conv3x3_halo /
 *              dp_conv3x3_halo_packed); must not overlap y_patch or ws
 * Other arguments, requirements and errors as dp_conv3x3_halo; w_packed other
 * than 0 or 1 gives DP_ERR_ARG.
 * ---------------------------------------------------------------------- */
dp_status dp_conv3x3_halo_residual(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                                   const void* x_stale, const void* w, int32_t w_packed, const float* bias,
                                   const void* residual, void* y_patch, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_groupnorm_conv3x3_halo -- GroupNorm (+SiLU) of patch i, then the 3x3
 * conv with stale halo on the normalised band, which also replaces band i of
 * the conv's stale map: the three calls
 *   dp_groupnorm_async(x_patch -> u_patch)
 *   dp_stale_update(u_patch -> band i of u_stale)
 *   dp_conv3x3_halo_residual(u_patch, u_stale -> y_patch)
 * in one, with bitwise the same results (u_stale, y_patch, fresh_stats_out).
 *
 * Source: the GroupNorm as dp_groupnorm_async (DistriFusion summary on
 * atlas.scime.ai, Approach) feeding the convolution of dp_conv3x3_halo
 * (study.space page, Method): in the denoiser's ResNet blocks a GroupNorm and
 * its activation precede every 3x3 conv, and the normalised band is what the
 * next step's halo rows come from.  Where the 256x160-tile conv runs (bf16,
 * large bands) the normalisation is folded into the conv's operand loads: the
 * band is read once raw (statistics) and once by the conv, and the normalised
 * band is never read back from memory.  Other shapes run the three kernels.
 *
 *   x_patch         [B][h][W][C] dtype, the GroupNorm input band
 *   stale_stats, gamma, beta, fresh_stats_out, G, eps, mode, act
 *                   as dp_groupnorm_async (fresh_stats_out may be slot i of
 *                   stale_stats in DP_GN_CORRECTED mode)
 *   u_stale         [B][H][W][C] dtype, the conv input's stale map (the
 *                   previous step's normalised map); band i is overwritten
 *                   with this step's normalised band, other rows only read
 *   Cout, w, w_packed, bias, residual
 *                   as dp_conv3x3_halo_residual (residual may be NULL)
 *   y_patch         [B][h][W][Cout] dtype
 *   ws              >= dp_groupnorm_conv3x3_halo_ws bytes
 * No written buffer (u_stale, y_patch, fresh_stats_out, ws) may overlap
 * another buffer of the call, except the slot-i case above.  Requirements
 * and errors are those of dp_groupnorm_async and dp_conv3x3_halo together
 * (y_patch is required); nothing is enqueued when a check fails.
 * ---------------------------------------------------------------------- */
dp_status dp_groupnorm_conv3x3_halo_ws(const dp_patch* p, dp_dtype dtype, int32_t G, int32_t Cout,
                                       size_t* ws_bytes);

dp_status dp_groupnorm_conv3x3_halo(const dp_patch* p, dp_dtype dtype, int32_t G, float eps, dp_gn_mode mode,
                                    dp_act act, const void* x_patch, const float* stale_stats, const float* gamma,
                                    const float* beta, float* fresh_stats_out, void* u_stale, int32_t Cout,
                                    const void* w, int32_t w_packed, const float* bias, const void* residual,
                                    void* y_patch, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_attention_splice -- self-attention of patch i over spliced K/V.
 *
 * Source: PipeFusion explainer (gist.science), Problem Statement and Memory
 * Efficiency: DistriFusion keeps the full spatial K and V of every layer on
 * every device; with the study.space Method (stale context, fresh patch).
 * Reading: for head e (channels [e*d, (e+1)*d)) and query token q of the band,
 *   O[q] = sum_n softmax_n(scale * <Q[q], K[n]>) V[n]
 * with K[n] = k_patch[n - r0*W] for tokens n of the band [r0*W, (r0+h)*W) and
 * k_stale[n] elsewhere; likewise V.  No mask.  scale <= 0 selects d^-1/2.
 *
 *   q_patch, k_patch, v_patch  [B][h*W][heads*head_dim] dtype
 *   k_stale, v_stale           [B][H*W][heads*head_dim] dtype
 *   o_patch                    [B][h*W][heads*head_dim] dtype; must not
 *                              overlap any input
 * k_patch / v_patch may point into band i of k_stale / v_stale (an in-place
 * splice done before the call); the result is the same.
 * Requires heads*head_dim == p->C and H*W < 2^31 tokens.  bf16: head_dim ==
 * 64.  f32: head_dim in {4, 8, 16, 32, 64, 128}.  Other head sizes give
 * DP_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
dp_status dp_attention_splice_ws(const dp_patch* p, dp_dtype dtype, int32_t heads,
                                 int32_t head_dim, size_t* ws_bytes);

dp_status dp_attention_splice(const dp_patch* p, dp_dtype dtype, int32_t heads, int32_t head_dim,
                              float scale, const void* q_patch, const void* k_patch,
                              const void* v_patch, const void* k_stale, const void* v_stale,
                              void* o_patch, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_stale_update -- write the fresh patch into the resident stale map.
 *
 * Source: DistriFusion summary (atlas.scime.ai), Approach (the AllGather of
 * fresh activations that becomes the next step's context); study.space page,
 * Method.  On one GPU this is the own-band part of what the gather delivers:
 *   stale[b, r0:r0+h, :, :] = x_patch[b]   bit for bit; other rows untouched.
 *
 *   x_patch  [B][h][W][C] dtype
 *   stale    [B][H][W][C] dtype, updated in place
 * x_patch may be band i of stale itself (then nothing is done); any other
 * overlap is an error.  The GroupNorm statistics table [P][B][G][2] is updated
 * with the same call viewed as a map: dtype DP_F32, B=1, H=P, W=1,
 * C=B*G*2, P=P, i=i, x_patch = fresh_stats_out.
 * ---------------------------------------------------------------------- */
dp_status dp_stale_update(const dp_patch* p, dp_dtype dtype, const void* x_patch, void* stale,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_linear -- y = x W^T + bias: the learned projections of an attention layer.
 *
 * Source: PipeFusion explainer (gist.science), Problem Statement and Memory
 * Efficiency: every device keeps the full spatial K and V of every layer; with
 * learned projections those are the projected keys and values, so a patch
 * projects its own tokens (Q, K, V = h W^T + b) and writes its fresh K and V
 * into band i of the cached maps, then projects the attention output by W_o.
 *
 *   x     [M][K] dtype, row r at x + r*ldx (elements)
 *   w     [N][K] dtype, contiguous
 *   bias  [N] float or NULL (0)
 *   y     [M][N] dtype, row r at y + r*ldy; must not overlap x, w or bias
 *         (a band of a token-major map [B][H*W][C] with B == 1 is M = h*W rows
 *         with ldy = C, so K and V can be written straight into the cache)
 * M may be 0 (nothing is enqueued; x and y may then be NULL).  bf16: K % 64 == 0, N, ldx, ldy multiples
 * of 8; fp32 accumulate, outputs rounded to nearest even.  f32: any K, N.
 * No workspace.
 * ---------------------------------------------------------------------- */
dp_status dp_linear(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w,
                    const float* bias, void* y, int64_t ldy, hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_linear_residual -- y = x W^T + bias + r: dp_linear with a residual added
 * in fp32 before the single rounding of the output.
 *
 * Source: as dp_linear (PipeFusion explainer on gist.science, Problem
 * Statement); the residual is the skip connection of a transformer block of
 * the U-Net denoiser (AsyncDiff rebuttal on paperhub.cn, answer to Q2): the
 * output projection of the attention adds the block input of the same tokens.
 *
 *   r     [M][N] dtype, row r at r + m*ldr (elements), or NULL (then exactly
 *         dp_linear); must not overlap y
 * Other arguments, requirements and errors as dp_linear; bf16 also needs ldr
 * a multiple of 8, and ldr >= N when r is given.
 * ---------------------------------------------------------------------- */
dp_status dp_linear_residual(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx,
                             const void* w, const float* bias, const void* r, int64_t ldr, void* y, int64_t ldy,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * dp_linear_qkv -- the three input projections of an attention layer in one
 * launch:  y_s = x W_s^T + bias_s  for s = Q, K, V, with W_s rows [s*N, (s+1)*N)
 * of w3 and bias_s entries [s*N, (s+1)*N) of bias3.  Bitwise equal to three
 * dp_linear calls; one product [M][3N] fills the GPU where three [M][N]
 * products of a small band would each leave it part idle.
 *
 * Source: as dp_linear (PipeFusion explainer on gist.science, Problem
 * Statement and Memory Efficiency: a patch projects its own tokens to Q, K
 * and V and writes the fresh K and V into band i of the cached maps).
 *
 *   x           [M][K] dtype, row r at x + r*ldx
 *   w3          [3N][K] dtype, contiguous (W_q, W_k, W_v stacked)
 *   bias3       [3N] float or NULL (0)
 *   yq, yk, yv  [M][N] dtype, row r at y + r*ld (ldq, ldk, ldv); none may
 *               overlap x, w3, bias3 or another output
 * Requirements and errors as dp_linear (bf16: every row stride a multiple of
 * 8).  No workspace.
 * ---------------------------------------------------------------------- */
dp_status dp_linear_qkv(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w3,
                        const float* bias3, void* yq, int64_t ldq, void* yk, int64_t ldk, void* yv, int64_t ldv,
                        hipStream_t stream);

/* Description of the last error on the calling thread (empty if none). The
 * string stays valid until the thread's next dp_* call. */
const char* dp_last_error(void);

/* Library version string. */
const char* dp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DP_H */
