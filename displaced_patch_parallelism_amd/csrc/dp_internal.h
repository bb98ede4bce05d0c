// Internal interface between the host entry points (dp_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dp {

// A 1-D grid of n blocks is launchable (at most 2^31 - 1 blocks); launches return
// hipErrorInvalidConfiguration otherwise, never a truncated grid.
inline bool grid_fits(int64_t n) { return n >= 1 && n <= 0x7fffffffLL; }

// Geometry of one patch of an NHWC map split into P equal row bands.
struct Geom {
    int B, H, W, C, P, i;
    int h;   // rows per band
    int r0;  // first row of band i
    int64_t band_tokens() const { return (int64_t)h * W; }   // per batch
    int64_t map_tokens() const { return (int64_t)H * W; }    // per batch
};

// ---- band splice --------------------------------------------------------
hipError_t launch_band_copy(const void* src, void* dst, const Geom& g, size_t elem_bytes,
                            hipStream_t stream);

// ---- GroupNorm ---------------------------------------------------------
struct GnPlan {
    int vec;          // elements per 16-byte vector
    int vpt;          // vectors per token (C / vec)
    int rows;         // tokens a normalising block reads in parallel
    int threads;      // normalising block size = vpt * rows (>= G)
    int rows_stats;   // tokens a statistics block reads in parallel (<= rows)
    int threads_stats;  // statistics block size = vpt * rows_stats
    int nblk;         // statistics blocks per batch
    int tok_per_blk;  // tokens per statistics block (the same split for every path, so the
                      // fresh moments are bitwise identical however they are computed)
    int nblk_apply;   // normalising blocks per batch
    int tpt_apply;    // token rows per normalising thread (4, or 2 or 1 for small bands)
    int tok_per_blk_apply;  // tokens per normalising block (rows * tpt_apply)
    size_t partial_floats;  // B * nblk * G * 2
    size_t ws_bytes;
};
GnPlan plan_groupnorm(const Geom& g, int G, bool bf16);
// Dynamic LDS bytes of the two GroupNorm kernels under a plan (the host rejects plans whose
// blocks exceed 1024 threads or whose LDS exceeds kMaxGnLds before anything is enqueued).
constexpr size_t kMaxGnLds = 64 * 1024;
size_t gn_stats_lds_bytes(const Geom& g, const GnPlan& plan);
size_t gn_apply_lds_bytes(const Geom& g, const GnPlan& plan, int G);
// Allocation-free GroupNorm: the statistics partials live in a static device array of this many
// bytes (one per GPU); groupnorm_scratch returns its address on the stream's device.
constexpr size_t kNoallocScratchBytes = (size_t)1 << 20;
hipError_t groupnorm_scratch(hipStream_t stream, void** out);
// The statistics pass alone: partials [nblk][B][G] (sum, sum of squares) into ws.
hipError_t launch_gn_stats(const Geom& g, const GnPlan& plan, bool bf16, int G, const void* x, void* ws,
                           hipStream_t stream);
// 1 / (elements of one group in the band), as both normalising paths scale the sums.
float gn_inv_count(const Geom& g, int G);
hipError_t launch_groupnorm(const Geom& g, const GnPlan& plan, bool bf16, int G, float eps, int mode,
                            int act, const void* x, const float* stale_stats, const float* gamma,
                            const float* beta, float* fresh_stats_out, void* y, void* ws,
                            hipStream_t stream);

// ---- conv3x3 with stale halo -------------------------------------------
struct ConvPlan {
    int kind;       // 0 = f32 direct, 1 = bf16 shared-ring 128x160 tiles, 2 = bf16 wave-split 64x80
                    // tiles, 3 = bf16 shared-ring 256x160 tiles (GroupNorm folded in only)
    int bm, bn;     // output tile (pixels x output channels)
    int mtiles, ntiles;
    int ktiles;     // K stages: 32 input channels of one kernel row each (3 * Cin / 32)
    int ksplit;     // K partitions (>1: fp32 partials + ordered reduction)
    size_t ws_bytes;
};
// gn_fused: plan for the conv with a GroupNorm folded into its A operand (the only user of the
// 256x160 tiles); else the standalone conv.
ConvPlan plan_conv(const Geom& g, int Cout, bool bf16, bool gn_fused = false);
// res: optional residual [B][h][W][Cout] added before the output is rounded.
hipError_t launch_conv(const Geom& g, const ConvPlan& plan, bool bf16, int Cout, const void* x_patch,
                       const void* x_stale, const void* w, bool w_packed, const float* bias, const void* res,
                       void* y, void* ws, hipStream_t stream);
// GroupNorm (+SiLU) folded into the 256x160-tile conv (plan kind 3): the conv's A operand is
// the raw GroupNorm input band x_patch, normalised on the fly with the band's statistics
// partials (launch_gn_stats, in ws) and the stale moments; the normalised band also goes to band
// i of u_stale, the conv's stale map.  conv_gn_fusable says whether a geometry takes this path.
bool conv_gn_fusable(const Geom& g, const ConvPlan& cp, const GnPlan& gp, int G, bool bf16);
hipError_t launch_conv_gn(const Geom& g, const ConvPlan& cp, const GnPlan& gp, int G, float eps, int mode, int act,
                          const void* x_patch, const float* stale_stats, const float* gamma, const float* beta,
                          float* fresh_stats_out, void* u_stale, int Cout, const void* w, bool w_packed,
                          const float* bias, const void* res, void* y, const void* gn_partials,
                          hipStream_t stream);
// bf16 weights [Cout][3][3][Cin] -> packed [3][Cin/32][3][Cout][32] (Cin % 32 == 0)
hipError_t launch_conv_pack(int Cin, int Cout, const void* w, void* w_packed, hipStream_t stream);

// ---- attention over spliced K/V ------------------------------------------
struct AttnPlan {
    int kind;       // 0 = f32 per-query, 1 = bf16 MFMA flash
    int qtile;      // queries per workgroup
    int qtiles;
    int kvsplit;    // key partitions (>1: partial results + log-sum-exp merge)
    size_t ws_bytes;
};
AttnPlan plan_attention(const Geom& g, int heads, int head_dim, bool bf16);
hipError_t launch_attention(const Geom& g, const AttnPlan& plan, bool bf16, int heads, int head_dim,
                            float scale, const void* q, const void* k, const void* v,
                            const void* k_stale, const void* v_stale, void* o, void* ws,
                            hipStream_t stream);

// ---- learned projections: y = x W^T + bias ----------------------------------
// r: optional residual [M][N] (row stride ldr) added before the output is rounded.
hipError_t launch_linear(bool bf16, int M, int N, int K, const void* x, int64_t ldx, const void* w,
                         const float* bias, const void* r, int64_t ldr, void* y, int64_t ldy,
                         hipStream_t stream);
// Q, K and V projections in one product: w3 [3N][K] (W_q, W_k, W_v stacked), bias3 [3N] or null;
// output segment s (columns s*N ..) goes to y[s] with row stride ldy[s].
hipError_t launch_linear_qkv(bool bf16, int M, int N, int K, const void* x, int64_t ldx, const void* w3,
                             const float* bias3, void* const y[3], const int64_t ldy[3], hipStream_t stream);

}  // namespace dp
