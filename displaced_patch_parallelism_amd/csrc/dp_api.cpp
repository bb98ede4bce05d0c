// Host entry points of the C ABI declared in include/dp.h: argument
// validation, plan selection and kernel dispatch.  Validation touches no HIP
// API, so a rejected call never initialises the runtime or enqueues work.

#include "dp.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dp_internal.h"

namespace {

thread_local std::string g_err;

dp_status fail(dp_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

dp_status ok() {
    g_err.clear();
    return DP_OK;
}

dp_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

size_t elem_size(dp_dtype dt) { return dt == DP_BF16 ? 2 : 4; }

// [a, a+na) and [b, b+nb) intersect
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Validates the patch geometry; fills g.
dp_status check_patch(const dp_patch* p, dp_dtype dt, dp::Geom* g) {
    if (!p) return fail(DP_ERR_ARG, "patch descriptor is NULL");
    if (dt != DP_F32 && dt != DP_BF16) return fail(DP_ERR_ARG, "unknown dtype %d", (int)dt);
    if (p->B < 1 || p->H < 1 || p->W < 1 || p->C < 1 || p->P < 1)
        return fail(DP_ERR_ARG, "B, H, W, C and P must be >= 1 (got B=%d H=%d W=%d C=%d P=%d)",
                    p->B, p->H, p->W, p->C, p->P);
    if (p->H % p->P != 0) return fail(DP_ERR_ARG, "H=%d is not divisible by P=%d", p->H, p->P);
    if (p->i < 0 || p->i >= p->P) return fail(DP_ERR_ARG, "patch index i=%d not in [0, %d)", p->i, p->P);
    const int64_t elems = (int64_t)p->B * p->H * p->W * p->C;
    if (elems > ((int64_t)1 << 40)) return fail(DP_ERR_ARG, "map too large");
    if (p->B > 65535) return fail(DP_ERR_UNSUPPORTED, "B=%d exceeds 65535 (the batch is a grid dimension)", p->B);
    g->B = p->B; g->H = p->H; g->W = p->W; g->C = p->C; g->P = p->P; g->i = p->i;
    g->h = p->H / p->P;
    g->r0 = p->i * g->h;
    return DP_OK;
}

#define DP_TRY(expr)                      \
    do {                                  \
        dp_status _s = (expr);            \
        if (_s != DP_OK) return _s;       \
    } while (0)

#define DP_NEED(ptr, name)                                                  \
    do {                                                                    \
        if (!(ptr)) return fail(DP_ERR_ARG, "%s is NULL", name);            \
        if (!aligned16(ptr)) return fail(DP_ERR_ARG, "%s is not 16-byte aligned", name); \
    } while (0)

#define DP_OPT(ptr, name)                                                   \
    do {                                                                    \
        if ((ptr) && !aligned16(ptr))                                       \
            return fail(DP_ERR_ARG, "%s is not 16-byte aligned", name);     \
    } while (0)

// ---- GroupNorm -----------------------------------------------------------

dp_status check_gn(const dp_patch* p, dp_dtype dt, int32_t G, dp::Geom* g) {
    DP_TRY(check_patch(p, dt, g));
    if (G < 1 || g->C % G != 0) return fail(DP_ERR_ARG, "C=%d is not divisible by G=%d", g->C, G);
    const int vec = dt == DP_BF16 ? 8 : 4;
    if (g->C % vec != 0)
        return fail(DP_ERR_UNSUPPORTED, "GroupNorm needs C %% %d == 0 for this dtype (C=%d)", vec, g->C);
    // a block holds one thread per 16-byte channel vector of a token: at most 1024 of them
    if (g->C / vec > 1024)
        return fail(DP_ERR_UNSUPPORTED, "GroupNorm supports C <= %d for this dtype (C=%d)", 1024 * vec, g->C);
    // the normalising block holds at least one thread per group, and both kernels' blocks must
    // fit 1024 threads and their LDS; rejected here, so nothing is enqueued
    const dp::GnPlan plan = dp::plan_groupnorm(*g, G, dt == DP_BF16);
    if (G > 1024 || plan.threads > 1024 || plan.threads_stats > 1024 ||
        dp::gn_stats_lds_bytes(*g, plan) > dp::kMaxGnLds || dp::gn_apply_lds_bytes(*g, plan, G) > dp::kMaxGnLds)
        return fail(DP_ERR_UNSUPPORTED, "GroupNorm with G=%d groups over C=%d channels needs a block of more "
                    "than 1024 threads or more than 64 KB of LDS (G <= 1024 is required)", G, g->C);
    return DP_OK;
}

// ---- conv ------------------------------------------------------------------

dp_status check_conv(const dp_patch* p, dp_dtype dt, int32_t Cout, dp::Geom* g) {
    DP_TRY(check_patch(p, dt, g));
    if (Cout < 1) return fail(DP_ERR_ARG, "Cout=%d must be >= 1", Cout);
    if (dt == DP_BF16 && (g->C % 64 != 0 || Cout % 32 != 0))
        return fail(DP_ERR_UNSUPPORTED, "bf16 conv needs Cin %% 64 == 0 and Cout %% 32 == 0 (Cin=%d Cout=%d)",
                    g->C, Cout);
    // the bf16 kernels address one batch image and the weights with 32-bit offsets
    if (dt == DP_BF16 && ((int64_t)g->H * g->W * g->C >= (int64_t)1 << 31 ||
                          (int64_t)9 * g->C * Cout * 2 >= (int64_t)1 << 31 ||
                          (int64_t)g->B * g->h * g->W >= (int64_t)1 << 31))
        return fail(DP_ERR_UNSUPPORTED,
                    "bf16 conv needs H*W*Cin < 2^31 elements, weights < 2 GiB and B*h*W < 2^31 output pixels");
    return DP_OK;
}

// ---- attention ---------------------------------------------------------------

dp_status check_attn(const dp_patch* p, dp_dtype dt, int32_t heads, int32_t head_dim, dp::Geom* g) {
    DP_TRY(check_patch(p, dt, g));
    if (heads < 1 || head_dim < 1) return fail(DP_ERR_ARG, "heads and head_dim must be >= 1");
    if ((int64_t)heads * head_dim != g->C)
        return fail(DP_ERR_ARG, "heads*head_dim=%d does not equal C=%d", heads * head_dim, g->C);
    if ((int64_t)g->H * g->W >= ((int64_t)1 << 31))
        return fail(DP_ERR_UNSUPPORTED, "attention needs H*W < 2^31 tokens (H=%d W=%d)", g->H, g->W);
    if (dt == DP_BF16 && head_dim != 64)
        return fail(DP_ERR_UNSUPPORTED, "bf16 attention is built for head_dim 64 (got %d)", head_dim);
    if (dt == DP_F32 && !(head_dim == 4 || head_dim == 8 || head_dim == 16 || head_dim == 32 ||
                          head_dim == 64 || head_dim == 128))
        return fail(DP_ERR_UNSUPPORTED, "f32 attention is built for head_dim in {4,8,16,32,64,128} (got %d)",
                    head_dim);
    return DP_OK;
}

}  // namespace

extern "C" {

const char* dp_last_error(void) { return g_err.c_str(); }

const char* dp_version(void) { return "dp 0.1 (gfx950)"; }

dp_status dp_stale_update(const dp_patch* p, dp_dtype dtype, const void* x_patch, void* stale,
                          hipStream_t stream) {
    dp::Geom g;
    DP_TRY(check_patch(p, dtype, &g));
    DP_NEED(x_patch, "x_patch");
    DP_NEED(stale, "stale");
    const size_t es = elem_size(dtype);
    const size_t band_bytes = (size_t)g.B * g.band_tokens() * g.C * es;
    const size_t map_bytes = (size_t)g.B * g.map_tokens() * g.C * es;
    const char* band_i = (const char*)stale + (size_t)g.r0 * g.W * g.C * es;
    if (g.B == 1 && x_patch == (const void*)band_i) return ok();  // already in place
    if (overlaps(x_patch, band_bytes, stale, map_bytes))
        return fail(DP_ERR_ARG, "x_patch overlaps the stale map (other than being band i itself)");
    return hip_status(dp::launch_band_copy(x_patch, stale, g, es, stream), "dp_stale_update launch");
}

dp_status dp_groupnorm_async_ws(const dp_patch* p, dp_dtype dtype, int32_t G, size_t* ws_bytes) {
    dp::Geom g;
    DP_TRY(check_gn(p, dtype, G, &g));
    if (!ws_bytes) return fail(DP_ERR_ARG, "ws_bytes is NULL");
    *ws_bytes = dp::plan_groupnorm(g, G, dtype == DP_BF16).ws_bytes;
    return ok();
}

}  // extern "C"

namespace {

// Validation and launch shared by dp_groupnorm_async and dp_groupnorm_async_noalloc; `noalloc`
// takes the statistics partials' scratch from the library's static array instead of ws.
dp_status groupnorm_call(const dp_patch* p, dp_dtype dtype, int32_t G, float eps, dp_gn_mode mode, dp_act act,
                         const void* x_patch, const float* stale_stats, const float* gamma, const float* beta,
                         float* fresh_stats_out, void* y_patch, void* ws, size_t ws_bytes, bool noalloc,
                         hipStream_t stream) {
    dp::Geom g;
    DP_TRY(check_gn(p, dtype, G, &g));
    if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(DP_ERR_ARG, "eps must be a positive finite number");
    if (mode != DP_GN_CORRECTED && mode != DP_GN_LOCAL && mode != DP_GN_STALE)
        return fail(DP_ERR_ARG, "unknown GroupNorm mode %d", (int)mode);
    if (act != DP_ACT_NONE && act != DP_ACT_SILU) return fail(DP_ERR_ARG, "unknown activation %d", (int)act);
    DP_NEED(x_patch, "x_patch");
    DP_OPT(gamma, "gamma");
    DP_OPT(beta, "beta");
    DP_OPT(fresh_stats_out, "fresh_stats_out");
    DP_OPT(y_patch, "y_patch");
    if (!y_patch && !fresh_stats_out)
        return fail(DP_ERR_ARG, "nothing to compute: y_patch and fresh_stats_out are both NULL");
    if (y_patch && mode != DP_GN_LOCAL && !stale_stats)
        return fail(DP_ERR_ARG, "stale_stats is NULL (needed by this GroupNorm mode)");
    DP_OPT(stale_stats, "stale_stats");
    const dp::GnPlan plan = dp::plan_groupnorm(g, G, dtype == DP_BF16);
    if (noalloc) {
        if (plan.ws_bytes > dp::kNoallocScratchBytes)
            return fail(DP_ERR_UNSUPPORTED, "dp_groupnorm_async_noalloc: this call needs %zu bytes of scratch, "
                        "more than the %zu its static array holds (use dp_groupnorm_async with a workspace)",
                        plan.ws_bytes, dp::kNoallocScratchBytes);
        ws = nullptr;
        ws_bytes = 0;
    } else {
        if (ws_bytes < plan.ws_bytes)
            return fail(DP_ERR_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, plan.ws_bytes);
        DP_NEED(ws, "ws");
    }
    const size_t es = elem_size(dtype);
    const size_t band_bytes = (size_t)g.B * g.band_tokens() * g.C * es;
    const size_t stats_bytes = (size_t)g.B * G * 2 * sizeof(float);
    const size_t table_bytes = (size_t)g.P * stats_bytes;
    if (y_patch && y_patch != x_patch && overlaps(y_patch, band_bytes, x_patch, band_bytes))
        return fail(DP_ERR_ARG, "y_patch partially overlaps x_patch");
    if (y_patch && (overlaps(y_patch, band_bytes, stale_stats, table_bytes) ||
                    overlaps(y_patch, band_bytes, ws, plan.ws_bytes)))
        return fail(DP_ERR_ARG, "y_patch overlaps the statistics table or the workspace");
    // fresh_stats_out may be slot i of the table in CORRECTED mode, which never reads slot i
    const bool stats_in_slot_i = stale_stats && mode == DP_GN_CORRECTED &&
                                 fresh_stats_out == stale_stats + (size_t)g.i * g.B * G * 2;
    if (fresh_stats_out && (overlaps(fresh_stats_out, stats_bytes, x_patch, band_bytes) ||
                            (!stats_in_slot_i && overlaps(fresh_stats_out, stats_bytes, stale_stats, table_bytes)) ||
                            overlaps(fresh_stats_out, stats_bytes, y_patch, band_bytes) ||
                            overlaps(fresh_stats_out, stats_bytes, ws, plan.ws_bytes)))
        return fail(DP_ERR_ARG, "fresh_stats_out overlaps an input, y_patch or the workspace");
    if (overlaps(ws, plan.ws_bytes, x_patch, band_bytes) || overlaps(ws, plan.ws_bytes, stale_stats, table_bytes))
        return fail(DP_ERR_ARG, "workspace overlaps an input");
    if (noalloc) {
        const hipError_t e = dp::groupnorm_scratch(stream, &ws);
        if (e != hipSuccess) return hip_status(e, "dp_groupnorm_async_noalloc scratch address");
    }
    return hip_status(dp::launch_groupnorm(g, plan, dtype == DP_BF16, G, eps, (int)mode, (int)act, x_patch,
                                           stale_stats, gamma, beta, fresh_stats_out, y_patch, ws, stream),
                      noalloc ? "dp_groupnorm_async_noalloc launch" : "dp_groupnorm_async launch");
}

}  // namespace

extern "C" {

dp_status dp_groupnorm_async(const dp_patch* p, dp_dtype dtype, int32_t G, float eps, dp_gn_mode mode,
                             dp_act act, const void* x_patch, const float* stale_stats,
                             const float* gamma, const float* beta, float* fresh_stats_out,
                             void* y_patch, void* ws, size_t ws_bytes, hipStream_t stream) {
    return groupnorm_call(p, dtype, G, eps, mode, act, x_patch, stale_stats, gamma, beta, fresh_stats_out,
                          y_patch, ws, ws_bytes, false, stream);
}

dp_status dp_groupnorm_async_noalloc(const dp_patch* p, dp_dtype dtype, int32_t G, float eps, dp_gn_mode mode,
                                     dp_act act, const void* x_patch, const float* stale_stats,
                                     const float* gamma, const float* beta, float* fresh_stats_out,
                                     void* y_patch, hipStream_t stream) {
    return groupnorm_call(p, dtype, G, eps, mode, act, x_patch, stale_stats, gamma, beta, fresh_stats_out,
                          y_patch, nullptr, 0, true, stream);
}

dp_status dp_conv3x3_halo_ws(const dp_patch* p, dp_dtype dtype, int32_t Cout, size_t* ws_bytes) {
    dp::Geom g;
    DP_TRY(check_conv(p, dtype, Cout, &g));
    if (!ws_bytes) return fail(DP_ERR_ARG, "ws_bytes is NULL");
    *ws_bytes = dp::plan_conv(g, Cout, dtype == DP_BF16).ws_bytes;
    return ok();
}

}  // extern "C"

namespace {

dp_status conv_call(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch, const void* x_stale,
                    const void* w, bool w_packed, const float* bias, const void* residual, void* y_patch,
                    void* ws, size_t ws_bytes, hipStream_t stream, const char* name) {
    dp::Geom g;
    DP_TRY(check_conv(p, dtype, Cout, &g));
    if (w_packed && dtype != DP_BF16) return fail(DP_ERR_UNSUPPORTED, "%s: packed weights are bf16 only", name);
    DP_NEED(x_patch, "x_patch");
    DP_NEED(x_stale, "x_stale");
    DP_NEED(w, w_packed ? "w_packed" : "w");
    DP_OPT(bias, "bias");
    DP_OPT(residual, "residual");
    DP_NEED(y_patch, "y_patch");
    const dp::ConvPlan plan = dp::plan_conv(g, Cout, dtype == DP_BF16);
    if (ws_bytes < plan.ws_bytes)
        return fail(DP_ERR_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, plan.ws_bytes);
    if (plan.ws_bytes) DP_NEED(ws, "ws");
    const size_t es = elem_size(dtype);
    const size_t in_band = (size_t)g.B * g.band_tokens() * g.C * es;
    const size_t in_map = (size_t)g.B * g.map_tokens() * g.C * es;
    const size_t out_band = (size_t)g.B * g.band_tokens() * Cout * es;
    const size_t w_bytes = (size_t)Cout * 9 * g.C * es;
    if (overlaps(y_patch, out_band, x_patch, in_band) || overlaps(y_patch, out_band, x_stale, in_map) ||
        overlaps(y_patch, out_band, w, w_bytes) || overlaps(y_patch, out_band, bias, Cout * sizeof(float)) ||
        overlaps(y_patch, out_band, ws, plan.ws_bytes) || overlaps(y_patch, out_band, residual, out_band))
        return fail(DP_ERR_ARG, "y_patch overlaps an input or the workspace");
    if (plan.ws_bytes && (overlaps(ws, plan.ws_bytes, x_patch, in_band) || overlaps(ws, plan.ws_bytes, x_stale, in_map) ||
                          overlaps(ws, plan.ws_bytes, w, w_bytes) || overlaps(ws, plan.ws_bytes, residual, out_band)))
        return fail(DP_ERR_ARG, "workspace overlaps an input");
    return hip_status(dp::launch_conv(g, plan, dtype == DP_BF16, Cout, x_patch, x_stale, w, w_packed, bias,
                                      residual, y_patch, ws, stream),
                      name);
}

}  // namespace

extern "C" {

dp_status dp_conv3x3_halo(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                          const void* x_stale, const void* w, const float* bias, void* y_patch,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
    return conv_call(p, dtype, Cout, x_patch, x_stale, w, false, bias, nullptr, y_patch, ws, ws_bytes, stream,
                     "dp_conv3x3_halo launch");
}

size_t dp_conv3x3_packed_weights_bytes(int32_t Cin, int32_t Cout) {
    if (Cin < 1 || Cout < 1) return 0;
    return (size_t)Cout * 9 * Cin * 2;
}

dp_status dp_conv3x3_pack_weights(dp_dtype dtype, int32_t Cin, int32_t Cout, const void* w, void* w_packed,
                                  hipStream_t stream) {
    if (dtype != DP_BF16) return fail(DP_ERR_UNSUPPORTED, "dp_conv3x3_pack_weights: bf16 only");
    if (Cin < 1 || Cout < 1) return fail(DP_ERR_ARG, "Cin=%d Cout=%d must be >= 1", Cin, Cout);
    if (Cin % 64 != 0 || Cout % 32 != 0)
        return fail(DP_ERR_UNSUPPORTED, "packed weights need Cin %% 64 == 0 and Cout %% 32 == 0 (Cin=%d Cout=%d)",
                    Cin, Cout);
    DP_NEED(w, "w");
    DP_NEED(w_packed, "w_packed");
    const size_t bytes = dp_conv3x3_packed_weights_bytes(Cin, Cout);
    if (overlaps(w, bytes, w_packed, bytes)) return fail(DP_ERR_ARG, "w_packed overlaps w");
    return hip_status(dp::launch_conv_pack(Cin, Cout, w, w_packed, stream), "dp_conv3x3_pack_weights launch");
}

dp_status dp_conv3x3_halo_packed(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                                 const void* x_stale, const void* w_packed, const float* bias, void* y_patch,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
    return conv_call(p, dtype, Cout, x_patch, x_stale, w_packed, true, bias, nullptr, y_patch, ws, ws_bytes, stream,
                     "dp_conv3x3_halo_packed launch");
}

dp_status dp_conv3x3_halo_residual(const dp_patch* p, dp_dtype dtype, int32_t Cout, const void* x_patch,
                                   const void* x_stale, const void* w, int32_t w_packed, const float* bias,
                                   const void* residual, void* y_patch, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    if (w_packed != 0 && w_packed != 1) return fail(DP_ERR_ARG, "w_packed must be 0 or 1 (got %d)", w_packed);
    return conv_call(p, dtype, Cout, x_patch, x_stale, w, w_packed == 1, bias, residual, y_patch, ws, ws_bytes,
                     stream, "dp_conv3x3_halo_residual launch");
}

}  // extern "C"

namespace {

// Workspace of the GroupNorm + conv call.  Fused: the statistics partials.  Otherwise the
// GroupNorm output band (B > 1 only: a band of a batched map is not one contiguous block, so it
// is normalised into the workspace and then spliced; for B == 1 it is normalised straight into
// band i of the conv's stale map) followed by one region the statistics partials and then the
// conv's split-K partials use in turn.
struct GnConvLayout {
    bool fused;
    size_t band_off, band_bytes, part_off, part_bytes, total;
};

GnConvLayout gn_conv_layout(const dp::Geom& g, int G, int Cout, bool bf16, dp::GnPlan* gp, dp::ConvPlan* cp) {
    *gp = dp::plan_groupnorm(g, G, bf16);
    *cp = dp::plan_conv(g, Cout, bf16, true);
    GnConvLayout l{};
    l.fused = dp::conv_gn_fusable(g, *cp, *gp, G, bf16);
    if (!l.fused) *cp = dp::plan_conv(g, Cout, bf16);    // the three calls: the standalone conv's plan
    if (l.fused) {
        l.part_bytes = gp->ws_bytes;
    } else {
        l.band_bytes = g.B > 1 ? (size_t)g.B * g.band_tokens() * g.C * (bf16 ? 2 : 4) : 0;
        l.part_off = (l.band_bytes + 255) & ~(size_t)255;
        l.part_bytes = gp->ws_bytes > cp->ws_bytes ? gp->ws_bytes : cp->ws_bytes;
    }
    l.total = l.part_off + l.part_bytes;
    return l;
}

}  // namespace

extern "C" {

dp_status dp_groupnorm_conv3x3_halo_ws(const dp_patch* p, dp_dtype dtype, int32_t G, int32_t Cout,
                                       size_t* ws_bytes) {
    dp::Geom g;
    DP_TRY(check_gn(p, dtype, G, &g));
    DP_TRY(check_conv(p, dtype, Cout, &g));
    if (!ws_bytes) return fail(DP_ERR_ARG, "ws_bytes is NULL");
    dp::GnPlan gp;
    dp::ConvPlan cp;
    *ws_bytes = gn_conv_layout(g, G, Cout, dtype == DP_BF16, &gp, &cp).total;
    return ok();
}

dp_status dp_groupnorm_conv3x3_halo(const dp_patch* p, dp_dtype dtype, int32_t G, float eps, dp_gn_mode mode,
                                    dp_act act, const void* x_patch, const float* stale_stats, const float* gamma,
                                    const float* beta, float* fresh_stats_out, void* u_stale, int32_t Cout,
                                    const void* w, int32_t w_packed, const float* bias, const void* residual,
                                    void* y_patch, void* ws, size_t ws_bytes, hipStream_t stream) {
    dp::Geom g;
    DP_TRY(check_gn(p, dtype, G, &g));
    DP_TRY(check_conv(p, dtype, Cout, &g));
    if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(DP_ERR_ARG, "eps must be a positive finite number");
    if (mode != DP_GN_CORRECTED && mode != DP_GN_LOCAL && mode != DP_GN_STALE)
        return fail(DP_ERR_ARG, "unknown GroupNorm mode %d", (int)mode);
    if (act != DP_ACT_NONE && act != DP_ACT_SILU) return fail(DP_ERR_ARG, "unknown activation %d", (int)act);
    if (w_packed != 0 && w_packed != 1) return fail(DP_ERR_ARG, "w_packed must be 0 or 1 (got %d)", w_packed);
    if (w_packed && dtype != DP_BF16) return fail(DP_ERR_UNSUPPORTED, "packed weights are bf16 only");
    DP_NEED(x_patch, "x_patch");
    DP_NEED(u_stale, "u_stale");
    DP_NEED(w, w_packed ? "w_packed" : "w");
    DP_NEED(y_patch, "y_patch");
    DP_OPT(gamma, "gamma");
    DP_OPT(beta, "beta");
    DP_OPT(fresh_stats_out, "fresh_stats_out");
    DP_OPT(bias, "bias");
    DP_OPT(residual, "residual");
    if (mode != DP_GN_LOCAL && !stale_stats)
        return fail(DP_ERR_ARG, "stale_stats is NULL (needed by this GroupNorm mode)");
    DP_OPT(stale_stats, "stale_stats");
    dp::GnPlan gp;
    dp::ConvPlan cp;
    const GnConvLayout l = gn_conv_layout(g, G, Cout, dtype == DP_BF16, &gp, &cp);
    if (ws_bytes < l.total) return fail(DP_ERR_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, l.total);
    if (l.total) DP_NEED(ws, "ws");
    const size_t es = elem_size(dtype);
    const size_t band = (size_t)g.B * g.band_tokens() * g.C * es;
    const size_t map = (size_t)g.B * g.map_tokens() * g.C * es;
    const size_t out_band = (size_t)g.B * g.band_tokens() * Cout * es;
    const size_t w_bytes = (size_t)Cout * 9 * g.C * es;
    const size_t stats_bytes = (size_t)g.B * G * 2 * sizeof(float);
    const size_t table_bytes = (size_t)g.P * stats_bytes;
    const size_t ch_bytes = (size_t)g.C * sizeof(float);
    const size_t wsb = l.total;
    // written: u_stale (band i), y_patch, fresh_stats_out, ws; everything else is only read
    if (overlaps(u_stale, map, x_patch, band) || overlaps(u_stale, map, stale_stats, table_bytes) ||
        overlaps(u_stale, map, gamma, ch_bytes) || overlaps(u_stale, map, beta, ch_bytes) ||
        overlaps(u_stale, map, w, w_bytes) || overlaps(u_stale, map, bias, Cout * sizeof(float)) ||
        overlaps(u_stale, map, residual, out_band) || overlaps(u_stale, map, ws, wsb))
        return fail(DP_ERR_ARG, "u_stale overlaps an input or the workspace");
    if (overlaps(y_patch, out_band, x_patch, band) || overlaps(y_patch, out_band, u_stale, map) ||
        overlaps(y_patch, out_band, stale_stats, table_bytes) || overlaps(y_patch, out_band, gamma, ch_bytes) ||
        overlaps(y_patch, out_band, beta, ch_bytes) || overlaps(y_patch, out_band, w, w_bytes) ||
        overlaps(y_patch, out_band, bias, Cout * sizeof(float)) || overlaps(y_patch, out_band, residual, out_band) ||
        overlaps(y_patch, out_band, ws, wsb))
        return fail(DP_ERR_ARG, "y_patch overlaps an input, u_stale or the workspace");
    const bool stats_in_slot_i = stale_stats && mode == DP_GN_CORRECTED &&
                                 fresh_stats_out == stale_stats + (size_t)g.i * g.B * G * 2;
    if (fresh_stats_out && (overlaps(fresh_stats_out, stats_bytes, x_patch, band) ||
                            (!stats_in_slot_i && overlaps(fresh_stats_out, stats_bytes, stale_stats, table_bytes)) ||
                            overlaps(fresh_stats_out, stats_bytes, u_stale, map) ||
                            overlaps(fresh_stats_out, stats_bytes, y_patch, out_band) ||
                            overlaps(fresh_stats_out, stats_bytes, gamma, ch_bytes) ||
                            overlaps(fresh_stats_out, stats_bytes, beta, ch_bytes) ||
                            overlaps(fresh_stats_out, stats_bytes, w, w_bytes) ||
                            overlaps(fresh_stats_out, stats_bytes, bias, Cout * sizeof(float)) ||
                            overlaps(fresh_stats_out, stats_bytes, residual, out_band) ||
                            overlaps(fresh_stats_out, stats_bytes, ws, wsb)))
        return fail(DP_ERR_ARG, "fresh_stats_out overlaps an input, an output or the workspace");
    if (overlaps(ws, wsb, x_patch, band) || overlaps(ws, wsb, stale_stats, table_bytes) ||
        overlaps(ws, wsb, gamma, ch_bytes) || overlaps(ws, wsb, beta, ch_bytes) || overlaps(ws, wsb, w, w_bytes) ||
        overlaps(ws, wsb, bias, Cout * sizeof(float)) || overlaps(ws, wsb, residual, out_band))
        return fail(DP_ERR_ARG, "workspace overlaps an input");
    const bool bf16 = dtype == DP_BF16;
    char* wsc = (char*)ws;
    if (l.fused) {
        hipError_t e = dp::launch_gn_stats(g, gp, bf16, G, x_patch, wsc, stream);
        if (e == hipSuccess)
            e = dp::launch_conv_gn(g, cp, gp, G, eps, (int)mode, (int)act, x_patch, stale_stats, gamma, beta,
                                   fresh_stats_out, u_stale, Cout, w, w_packed == 1, bias, residual, y_patch, wsc,
                                   stream);
        return hip_status(e, "dp_groupnorm_conv3x3_halo launch");
    }
    // the three calls it stands for: GroupNorm into the conv's input band, the splice of that
    // band into u_stale (in place for B == 1), the conv
    void* u_band = g.B == 1 ? (void*)((char*)u_stale + (size_t)g.r0 * g.W * g.C * es) : (void*)(wsc + l.band_off);
    void* part = l.part_bytes ? (void*)(wsc + l.part_off) : nullptr;
    hipError_t e = dp::launch_groupnorm(g, gp, bf16, G, eps, (int)mode, (int)act, x_patch, stale_stats, gamma, beta,
                                        fresh_stats_out, u_band, part, stream);
    if (e == hipSuccess && g.B > 1) e = dp::launch_band_copy(u_band, u_stale, g, es, stream);
    if (e == hipSuccess)
        e = dp::launch_conv(g, cp, bf16, Cout, u_band, u_stale, w, w_packed == 1, bias, residual, y_patch, part,
                            stream);
    return hip_status(e, "dp_groupnorm_conv3x3_halo launch");
}

dp_status dp_attention_splice_ws(const dp_patch* p, dp_dtype dtype, int32_t heads, int32_t head_dim,
                                 size_t* ws_bytes) {
    dp::Geom g;
    DP_TRY(check_attn(p, dtype, heads, head_dim, &g));
    if (!ws_bytes) return fail(DP_ERR_ARG, "ws_bytes is NULL");
    *ws_bytes = dp::plan_attention(g, heads, head_dim, dtype == DP_BF16).ws_bytes;
    return ok();
}

dp_status dp_attention_splice(const dp_patch* p, dp_dtype dtype, int32_t heads, int32_t head_dim, float scale,
                              const void* q_patch, const void* k_patch, const void* v_patch,
                              const void* k_stale, const void* v_stale, void* o_patch, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    dp::Geom g;
    DP_TRY(check_attn(p, dtype, heads, head_dim, &g));
    if (!std::isfinite(scale)) return fail(DP_ERR_ARG, "scale must be finite");
    if (scale <= 0.0f) scale = 1.0f / std::sqrt((float)head_dim);
    DP_NEED(q_patch, "q_patch");
    DP_NEED(k_patch, "k_patch");
    DP_NEED(v_patch, "v_patch");
    DP_NEED(k_stale, "k_stale");
    DP_NEED(v_stale, "v_stale");
    DP_NEED(o_patch, "o_patch");
    const dp::AttnPlan plan = dp::plan_attention(g, heads, head_dim, dtype == DP_BF16);
    if (ws_bytes < plan.ws_bytes)
        return fail(DP_ERR_ARG, "workspace too small: %zu < %zu bytes", ws_bytes, plan.ws_bytes);
    if (plan.ws_bytes) DP_NEED(ws, "ws");
    const size_t es = elem_size(dtype);
    const size_t band = (size_t)g.B * g.band_tokens() * g.C * es;
    const size_t map = (size_t)g.B * g.map_tokens() * g.C * es;
    if (overlaps(o_patch, band, q_patch, band) || overlaps(o_patch, band, k_patch, band) ||
        overlaps(o_patch, band, v_patch, band) || overlaps(o_patch, band, k_stale, map) ||
        overlaps(o_patch, band, v_stale, map) || overlaps(o_patch, band, ws, plan.ws_bytes))
        return fail(DP_ERR_ARG, "o_patch overlaps an input or the workspace");
    if (plan.ws_bytes && (overlaps(ws, plan.ws_bytes, q_patch, band) || overlaps(ws, plan.ws_bytes, k_patch, band) ||
                          overlaps(ws, plan.ws_bytes, v_patch, band) || overlaps(ws, plan.ws_bytes, k_stale, map) ||
                          overlaps(ws, plan.ws_bytes, v_stale, map)))
        return fail(DP_ERR_ARG, "workspace overlaps an input");
    return hip_status(dp::launch_attention(g, plan, dtype == DP_BF16, heads, head_dim, scale, q_patch, k_patch,
                                           v_patch, k_stale, v_stale, o_patch, ws, stream),
                      "dp_attention_splice launch");
}

}  // extern "C"

namespace {

dp_status linear_call(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w,
                      const float* bias, const void* r, int64_t ldr, void* y, int64_t ldy, hipStream_t stream,
                      const char* name) {
    if (dtype != DP_F32 && dtype != DP_BF16) return fail(DP_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || N < 1 || K < 1) return fail(DP_ERR_ARG, "need M >= 0, N >= 1, K >= 1 (got %d, %d, %d)", M, N, K);
    if (ldx < K || ldy < N) return fail(DP_ERR_ARG, "row strides must cover a row (ldx=%lld K=%d ldy=%lld N=%d)",
                                        (long long)ldx, K, (long long)ldy, N);
    if (r && ldr < N) return fail(DP_ERR_ARG, "residual row stride must cover a row (ldr=%lld N=%d)",
                                  (long long)ldr, N);
    if ((int64_t)M * ldx > ((int64_t)1 << 40) || (int64_t)M * ldy > ((int64_t)1 << 40) ||
        (r && (int64_t)M * ldr > ((int64_t)1 << 40)))
        return fail(DP_ERR_ARG, "matrix too large");
    if (dtype == DP_BF16 && (K % 64 != 0 || N % 8 != 0 || ldx % 8 != 0 || ldy % 8 != 0 || (r && ldr % 8 != 0)))
        return fail(DP_ERR_UNSUPPORTED, "bf16 linear needs K %% 64 == 0 and N, ldx, ldy (and ldr) multiples of 8 "
                    "(K=%d N=%d ldx=%lld ldy=%lld)", K, N, (long long)ldx, (long long)ldy);
    if (M == 0) return ok();   // nothing to compute; x, y and r may be NULL
    DP_NEED(x, "x");
    DP_NEED(w, "w");
    DP_OPT(bias, "bias");
    DP_OPT(r, "residual");
    DP_NEED(y, "y");
    const size_t es = elem_size(dtype);
    const size_t xb = ((size_t)(M - 1) * ldx + K) * es;
    const size_t yb = ((size_t)(M - 1) * ldy + N) * es;
    const size_t rb = r ? ((size_t)(M - 1) * ldr + N) * es : 0;
    const size_t wb = (size_t)N * K * es;
    if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb) || overlaps(y, yb, bias, bias ? (size_t)N * 4 : 0) ||
        overlaps(y, yb, r, rb))
        return fail(DP_ERR_ARG, "y overlaps an input");
    return hip_status(dp::launch_linear(dtype == DP_BF16, M, N, K, x, ldx, w, bias, r, ldr, y, ldy, stream), name);
}

}  // namespace

extern "C" {

dp_status dp_linear(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w,
                    const float* bias, void* y, int64_t ldy, hipStream_t stream) {
    return linear_call(dtype, M, N, K, x, ldx, w, bias, nullptr, 0, y, ldy, stream, "dp_linear launch");
}

dp_status dp_linear_residual(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx,
                             const void* w, const float* bias, const void* r, int64_t ldr, void* y, int64_t ldy,
                             hipStream_t stream) {
    return linear_call(dtype, M, N, K, x, ldx, w, bias, r, ldr, y, ldy, stream, "dp_linear_residual launch");
}

dp_status dp_linear_qkv(dp_dtype dtype, int32_t M, int32_t N, int32_t K, const void* x, int64_t ldx, const void* w3,
                        const float* bias3, void* yq, int64_t ldq, void* yk, int64_t ldk, void* yv, int64_t ldv,
                        hipStream_t stream) {
    if (dtype != DP_F32 && dtype != DP_BF16) return fail(DP_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || N < 1 || K < 1) return fail(DP_ERR_ARG, "need M >= 0, N >= 1, K >= 1 (got %d, %d, %d)", M, N, K);
    if ((int64_t)3 * N > 0x7fffffffLL) return fail(DP_ERR_ARG, "3N exceeds the 32-bit range");
    void* const y[3] = {yq, yk, yv};
    const int64_t ld[3] = {ldq, ldk, ldv};
    const char* nm[3] = {"yq", "yk", "yv"};
    if (ldx < K) return fail(DP_ERR_ARG, "row stride ldx=%lld does not cover K=%d", (long long)ldx, K);
    for (int s = 0; s < 3; ++s)
        if (ld[s] < N) return fail(DP_ERR_ARG, "row stride of %s (%lld) does not cover N=%d", nm[s], (long long)ld[s], N);
    if ((int64_t)M * ldx > ((int64_t)1 << 40) || (int64_t)M * ldq > ((int64_t)1 << 40) ||
        (int64_t)M * ldk > ((int64_t)1 << 40) || (int64_t)M * ldv > ((int64_t)1 << 40))
        return fail(DP_ERR_ARG, "matrix too large");
    if (dtype == DP_BF16 && (K % 64 != 0 || N % 8 != 0 || ldx % 8 != 0 || ldq % 8 != 0 || ldk % 8 != 0 ||
                             ldv % 8 != 0))
        return fail(DP_ERR_UNSUPPORTED, "bf16 linear needs K %% 64 == 0 and N, ldx and the output row strides "
                    "multiples of 8 (K=%d N=%d)", K, N);
    if (M == 0) return ok();
    DP_NEED(x, "x");
    DP_NEED(w3, "w3");
    DP_OPT(bias3, "bias3");
    for (int s = 0; s < 3; ++s) {
        if (!y[s]) return fail(DP_ERR_ARG, "%s is NULL", nm[s]);
        if (!aligned16(y[s])) return fail(DP_ERR_ARG, "%s is not 16-byte aligned", nm[s]);
    }
    const size_t es = elem_size(dtype);
    const size_t xb = ((size_t)(M - 1) * ldx + K) * es;
    const size_t wb = (size_t)3 * N * K * es;
    const size_t bb = bias3 ? (size_t)3 * N * sizeof(float) : 0;
    size_t yb[3];
    for (int s = 0; s < 3; ++s) yb[s] = ((size_t)(M - 1) * ld[s] + N) * es;
    for (int s = 0; s < 3; ++s) {
        if (overlaps(y[s], yb[s], x, xb) || overlaps(y[s], yb[s], w3, wb) || overlaps(y[s], yb[s], bias3, bb))
            return fail(DP_ERR_ARG, "%s overlaps an input", nm[s]);
        for (int t = s + 1; t < 3; ++t)
            if (overlaps(y[s], yb[s], y[t], yb[t])) return fail(DP_ERR_ARG, "%s overlaps %s", nm[s], nm[t]);
    }
    return hip_status(dp::launch_linear_qkv(dtype == DP_BF16, M, N, K, x, ldx, w3, bias3, y, ld, stream),
                      "dp_linear_qkv launch");
}

}  // extern "C"
