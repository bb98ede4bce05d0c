// Corrected asynchronous GroupNorm of one patch.
//
// DistriFusion summary (atlas.scime.ai), Approach: the stale activations
// that displaced patches read would bias GroupNorm's statistics, so a
// corrected asynchronous GroupNorm fixes them; the "Measured effects" table
// lists the rejected alternatives (on-device statistics only, stale
// statistics only) and the exact but synchronising one.  The patch
// normalises with the moments of the spliced map: its fresh band moments
// (m_i, q_i) plus the previous step's moments of every other band, each
// band weighted 1/P; variance = E[x^2] - E[x]^2 clamped at 0.
//
// Two launches, both streaming the band [B][h*W][C] with 16-byte vectors.
// A block is vpt x R threads: thread (cv, r) owns channel vector cv (8 bf16
// or 4 f32 channels) and token rows r, r+R, ... of the block's range, so
// per-channel state stays in registers.
//   1. gn_stats: each thread sums one round of up to 8 token loads in flight (a band too
//      large for that takes whole rounds); fp32 per-channel sums, reduced through LDS in a
//      fixed order to per-group (sum, sum of squares) partials [block][B][G].  The band is cut
//      into as many blocks as a normalising block can sum partials in one round of loads (at
//      most 256), so even a small band spreads over the GPU.
//   2. gn_apply: each block owns 4 token rows per thread (one round; 2 or 1 rows for a band
//      too small to give 256 such blocks, so that it still spreads over the GPU).  It issues the loads
//      of its tokens and the stale moments first; then adds the statistics partials of its
//      batch (every partial load in flight at once, each lane summing its share in a fixed
//      order, lanes combined in order through LDS), loads gamma/beta, forms the fresh moments
//      (block 0 stores them), combines them with the stale table into (mean, rstd), and writes
//      y = x*scale + shift (+ SiLU) rounded to the storage type.
// LDS sums that run over a runtime count read 8 values ahead and add them in order, so the
// order of every floating-point sum is fixed by the geometry.
// The statistics split depends only on the geometry, so the fresh moments are
// bitwise identical whichever entry path computes them.  No atomics.


#include "dp_device.h"
#include "dp_gn_device.h"
#include "dp_internal.h"

#include <mutex>

// Scratch of the allocation-free GroupNorm entry point: the statistics partials of a call live
// here instead of in a caller workspace.  Every GPU the library runs on holds its own copy until
// the process ends; host code never names the array itself (in host code the name is a host-side
// stand-in, not a device address) but only the per-device address groupnorm_scratch() returns.
static __device__ __align__(256) unsigned char scratch[dp::kNoallocScratchBytes];

namespace dp {
namespace {


template <bool BF16>
__device__ __forceinline__ void to_f32(const uint4& v, float* f) {
    if (BF16) {
        unpack8(v, f);
    } else {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
}

// x0 += p[k*stride].x, x1 += p[k*stride].y (or the two float arrays) for k < n, in k order,
// with 8 reads in flight at a time (a plain loop waits out every LDS read).
__device__ __forceinline__ void sum_lds_in_order(const float* ps, const float* pq, int stride, int n, float& x0,
                                                 float& x1) {
    int k = 0;
    for (; k + 8 <= n; k += 8) {
        float ts[8], tq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            ts[u] = ps[(k + u) * stride];
            tq[u] = pq[(k + u) * stride];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            x0 += ts[u];
            x1 += tq[u];
        }
    }
    for (; k < n; ++k) {
        x0 += ps[k * stride];
        x1 += pq[k * stride];
    }
}

// partial[(blk*B + b)*G + g] = (sum x, sum x^2) over the block's tokens.
template <bool BF16>
__global__ void gn_stats_kernel(const void* __restrict__ x, int64_t tokens, int C, int G, int vpt, int rows,
                                int tok_per_blk, float2* __restrict__ partial) {
    constexpr int VEC = BF16 ? 8 : 4;
    extern __shared__ float sh[];  // [2][rows][C]
    const int tid = threadIdx.x;
    const int cv = tid % vpt;
    const int r = tid / vpt;
    const int b = blockIdx.y;
    const int64_t t0 = (int64_t)blockIdx.x * tok_per_blk;
    int64_t t1 = t0 + tok_per_blk;
    if (t1 > tokens) t1 = tokens;

    float s[VEC], q[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[e] = q[e] = 0.f;
    const uint4* xb = (const uint4*)x + (int64_t)b * tokens * vpt + cv;
    // rounds of 8 token rows per thread, all 8 loads in flight (rows past the end read as
    // zeros, which add nothing to either sum)
    // (one 64-bit base per round; the round's rows are 32-bit offsets of it, rows * vpt = the
    // block size apart, so the address arithmetic ahead of the first load stays short)
    const int step = rows * vpt;
    for (int64_t t = t0 + r; t < t1; t += 8 * rows) {
        const uint4* p = xb + t * vpt;
        const int64_t left = t1 - t;
        const int nrow = left < 8 * rows ? (int)left : 8 * rows;
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = u * rows < nrow ? p[u * step] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float f[VEC];
            to_f32<BF16>(v[u], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                s[e] += f[e];
                q[e] = fmaf(f[e], f[e], q[e]);
            }
        }
    }
    float* sh_s = sh;
    float* sh_q = sh + (size_t)rows * C;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        sh_s[r * C + cv * VEC + e] = s[e];
        sh_q[r * C + cv * VEC + e] = q[e];
    }
    __syncthreads();
    // per-channel totals over the rows, in row order; kept in row 0 (one row: already there)
    if (rows > 1) {
        for (int c = tid; c < C; c += blockDim.x) {
            float a = sh_s[c], aq = sh_q[c];
            sum_lds_in_order(sh_s + C + c, sh_q + C + c, C, rows - 1, a, aq);
            sh_s[c] = a;
            sh_q[c] = aq;
        }
        __syncthreads();
    }
    const int cg = C / G;
    for (int g = tid; g < G; g += blockDim.x) {
        float a = 0.f, aq = 0.f;
        sum_lds_in_order(sh_s + g * cg, sh_q + g * cg, 1, cg, a, aq);
        partial[((int64_t)blockIdx.x * gridDim.y + b) * G + g] = make_float2(a, aq);
    }
}


struct GnApplyArgs {
    const void* x;
    void* y;                 // null: moments only
    const float2* partial;   // [nblk][B][G]
    int nblk;                // statistics blocks per batch
    int64_t tokens;          // per batch
    int B, C, G, P, i, mode, vpt, rows, tok_per_blk;   // tok_per_blk: tokens per apply block
    float inv_count, eps;
    const float* stale;      // [P][B][G][2]
    const float* gamma;
    const float* beta;
    float* fresh_out;        // [B][G][2] or null
};

// Stale-table entries ([P][G] of one batch) an apply block parks in LDS (32 KB).
constexpr int kStaleLds = 4096;

// PR: partial loads in flight per lane (8, or 16 for blocks whose lanes sum more than 8).
// TPT: token rows per thread (4, or 2 or 1 for a band too small to give 256 blocks of 4).
// At most 80 VGPRs (6 waves per SIMD): three blocks of up to 512 threads per CU, so a band of
// ~768 blocks is resident at once (at 85 the 16-load instance held two, and a large band ran
// its blocks in two waves).
template <bool BF16, bool SILU, int PR, int TPT>
__global__ __attribute__((amdgpu_waves_per_eu(6))) void gn_apply_kernel(GnApplyArgs a) {
    constexpr int VEC = BF16 ? 8 : 4;
    extern __shared__ float2 gsh[];          // [lanes_per_g][G] partial sums, [G] (mean, rstd), [P][G] stale
    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int G = a.G;
    const int cv = tid % a.vpt;
    const int r = tid / a.vpt;
    const bool data = a.y != nullptr && r < a.rows;

    // (1) independent loads first: this thread's tokens and (one thread per group) the stale
    // moments the mode combines with the fresh ones
    const int64_t t0 = (int64_t)blockIdx.x * a.tok_per_blk + r;
    const int64_t base = (int64_t)b * a.tokens * a.vpt + cv;
    const uint4* xv = (const uint4*)a.x + base;
    uint4 v[TPT];
    if (data) {
        const int64_t t_end = (int64_t)(blockIdx.x + 1) * a.tok_per_blk < a.tokens
                                  ? (int64_t)(blockIdx.x + 1) * a.tok_per_blk : a.tokens;
#pragma unroll
        for (int u = 0; u < TPT; ++u)
            if (t0 + u * a.rows < t_end) v[u] = xv[(t0 + u * a.rows) * a.vpt];
    }
    // the stale table's [P][G] moments of this batch, one entry per thread (a table larger than
    // kStaleLds entries is summed from memory by the group threads instead); each entry is
    // parked in LDS after the partial loads, so no thread waits on it before they are issued
    const bool stale_lds = a.mode != 1 && (int64_t)a.P * G <= kStaleLds;
    const int PG = stale_lds ? a.P * G : 0;
    float2 stv = make_float2(0.f, 0.f);
    if (stale_lds && tid < PG)
        stv = *(const float2*)(a.stale + (((int64_t)(tid / G) * a.B + b) * G + tid % G) * 2);

    // (2) fresh moments: lane j0 of group g sums partials j0, j0+L, ... in order (PR loads in
    // flight), then the L lane sums are added in lane order
    const int L = blockDim.x / G;            // >= 1: the plan gives blocks of >= G threads
    if (tid < L * G) {
        const int g = tid % G, j0 = tid / G;
        float sa = 0.f, sq = 0.f;
        for (int jb = j0; jb < a.nblk; jb += PR * L) {
            float2 pv[PR];
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                const int j = jb + u * L;
                pv[u] = j < a.nblk ? a.partial[((int64_t)j * a.B + b) * G + g] : make_float2(0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < PR; ++u) {
                sa += pv[u].x;
                sq += pv[u].y;
            }
        }
        gsh[j0 * G + g] = make_float2(sa, sq);
    }
    float2* mr = gsh + L * G;
    float2* stl = mr + G;
    if (stale_lds) {
        if (tid < PG) stl[tid] = stv;
        for (int k = tid + blockDim.x; k < PG; k += blockDim.x)
            stl[k] = *(const float2*)(a.stale + (((int64_t)(k / G) * a.B + b) * G + k % G) * 2);
    }
    // gamma/beta (L2-resident, 16-byte vectors): issued here, so they hold no registers during
    // the partial loads and arrive while the lanes are combined
    float4 gv[VEC / 4], bv[VEC / 4];
#pragma unroll
    for (int e4 = 0; e4 < VEC / 4; ++e4) {
        gv[e4] = make_float4(1.f, 1.f, 1.f, 1.f);
        bv[e4] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (data && a.gamma) {
        const float4* gp = (const float4*)(a.gamma + cv * VEC);
#pragma unroll
        for (int e4 = 0; e4 < VEC / 4; ++e4) gv[e4] = gp[e4];
    }
    if (data && a.beta) {
        const float4* bp = (const float4*)(a.beta + cv * VEC);
#pragma unroll
        for (int e4 = 0; e4 < VEC / 4; ++e4) bv[e4] = bp[e4];
    }
    __syncthreads();
    if (tid < G) {
        const int g = tid;
        float sa = 0.f, sq = 0.f;
        const float* gf = (const float*)gsh;     // float2 [L][G] as floats: x at 2k, y at 2k+1
        sum_lds_in_order(gf + 2 * g, gf + 2 * g + 1, 2 * G, L, sa, sq);
        // sum of the other bands' stale moments, in band order
        float st_e = 0.f, st_q = 0.f;
        if (stale_lds) {
            for (int j0 = 0; j0 < a.P; j0 += 8) {
                float2 t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = j0 + u < a.P ? stl[(j0 + u) * G + g] : make_float2(0.f, 0.f);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u;
                    if (j < a.P && !(a.mode == 0 && j == a.i)) {
                        st_e += t[u].x;
                        st_q += t[u].y;
                    }
                }
            }
        } else if (a.mode != 1) {
            for (int j = 0; j < a.P; ++j) {
                if (a.mode == 0 && j == a.i) continue;
                st_e += a.stale[((int64_t)j * a.B + b) * G * 2 + g * 2 + 0];
                st_q += a.stale[((int64_t)j * a.B + b) * G * 2 + g * 2 + 1];
            }
        }
        const float m = sa * a.inv_count, qm = sq * a.inv_count;
        if (a.fresh_out && blockIdx.x == 0) {
            a.fresh_out[(b * G + g) * 2 + 0] = m;
            a.fresh_out[(b * G + g) * 2 + 1] = qm;
        }
        mr[g] = gn_group_norm_params(m, qm, st_e, st_q, a.mode, a.P, a.eps);
    }
    if (!a.y) return;
    __syncthreads();
    if (!data) return;

    // (3) normalise: the tokens loaded in (1), then the block's further rounds of 4 rows
    const int cg = a.C / G;
    float ga[VEC], be[VEC];
#pragma unroll
    for (int e4 = 0; e4 < VEC / 4; ++e4) {
        ga[4 * e4 + 0] = gv[e4].x; ga[4 * e4 + 1] = gv[e4].y; ga[4 * e4 + 2] = gv[e4].z; ga[4 * e4 + 3] = gv[e4].w;
        be[4 * e4 + 0] = bv[e4].x; be[4 * e4 + 1] = bv[e4].y; be[4 * e4 + 2] = bv[e4].z; be[4 * e4 + 3] = bv[e4].w;
    }
    float sc[VEC], sf[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) gn_scale_shift(mr[(cv * VEC + e) / cg], ga[e], be[e], sc[e], sf[e]);
    uint4* yv = (uint4*)a.y + base;
    const int64_t t_end = (int64_t)(blockIdx.x + 1) * a.tok_per_blk < a.tokens
                              ? (int64_t)(blockIdx.x + 1) * a.tok_per_blk : a.tokens;
    for (int64_t tr = t0;; tr += TPT * a.rows) {
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int64_t t = tr + u * a.rows;
            if (t >= t_end) continue;
            float f[VEC];
            to_f32<BF16>(v[u], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float z = fmaf(f[e], sc[e], sf[e]);
                if (SILU) z = silu(z);
                f[e] = z;
            }
            uint4 o;
            if (BF16) o = pack8(f);
            else o = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
            yv[t * a.vpt] = o;
        }
        const int64_t tn = tr + TPT * a.rows;
        if (tn >= t_end) break;
#pragma unroll
        for (int u = 0; u < TPT; ++u)
            if (tn + u * a.rows < t_end) v[u] = xv[(tn + u * a.rows) * a.vpt];
    }
}

template <bool BF16, bool SILU>
hipError_t launch_gn_typed(const Geom& g, const GnPlan& plan, GnApplyArgs a, float2* partial, hipStream_t stream) {
    // statistics over the plan's token split
    {
        dim3 grid((unsigned)plan.nblk, (unsigned)g.B);
        const size_t shmem = gn_stats_lds_bytes(g, plan);
        gn_stats_kernel<BF16><<<grid, plan.threads_stats, shmem, stream>>>(a.x, a.tokens, g.C, a.G, plan.vpt,
                                                                          plan.rows_stats,
                                                                    plan.tok_per_blk, partial);
    }
    // apply: one round of rows * tpt_apply tokens per block; a moments-only call runs one
    // block per batch
    a.tok_per_blk = plan.tok_per_blk_apply;
    const int64_t nb = a.y ? plan.nblk_apply : 1;
    const size_t shmem = gn_apply_lds_bytes(g, plan, a.G);
    const dim3 grid_a((unsigned)nb, (unsigned)g.B);
    const bool pr16 = plan.nblk > 8 * (plan.threads / a.G);
    if (plan.tpt_apply == 1) {
        if (pr16) gn_apply_kernel<BF16, SILU, 16, 1><<<grid_a, plan.threads, shmem, stream>>>(a);
        else gn_apply_kernel<BF16, SILU, 8, 1><<<grid_a, plan.threads, shmem, stream>>>(a);
    } else if (plan.tpt_apply == 2) {
        if (pr16) gn_apply_kernel<BF16, SILU, 16, 2><<<grid_a, plan.threads, shmem, stream>>>(a);
        else gn_apply_kernel<BF16, SILU, 8, 2><<<grid_a, plan.threads, shmem, stream>>>(a);
    } else {
        if (pr16) gn_apply_kernel<BF16, SILU, 16, 4><<<grid_a, plan.threads, shmem, stream>>>(a);
        else gn_apply_kernel<BF16, SILU, 8, 4><<<grid_a, plan.threads, shmem, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

size_t gn_stats_lds_bytes(const Geom& g, const GnPlan& plan) {
    return (size_t)2 * plan.rows_stats * g.C * sizeof(float);
}

size_t gn_apply_lds_bytes(const Geom& g, const GnPlan& plan, int G) {
    const size_t pg = (size_t)g.P * G;
    return ((size_t)(plan.threads / G) * G + G + (pg <= (size_t)kStaleLds ? pg : 0)) * sizeof(float2);
}

// Device address of `scratch` on the device `stream` runs on (the current device for the null
// stream), looked up once per device with that device current.  No allocation.
hipError_t groupnorm_scratch(hipStream_t stream, void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t d;
        e = hipStreamGetDevice(stream, &d);
        if (e != hipSuccess) return e;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

GnPlan plan_groupnorm(const Geom& g, int G, bool bf16) {
    GnPlan p{};
    p.vec = bf16 ? 8 : 4;
    p.vpt = g.C / p.vec;
    // R token rows per block; block = vpt * R threads (<= 512 when vpt <= 512)
    p.rows = p.vpt >= 512 ? 1 : 512 / p.vpt;
    p.threads = p.vpt * p.rows;
    if (p.threads < G) {          // the reduction uses at least one thread per group
        p.rows = (G + p.vpt - 1) / p.vpt;
        p.threads = p.vpt * p.rows;
    }
    const int64_t tokens = g.band_tokens();
    // Apply split: one round of 4 token rows per thread, so every block's loads are in flight
    // together (a whole band is a few MB to a few tens of MB); a band that gives fewer than 256
    // such blocks takes 2 or 1 rows per thread instead -- the most that still give 128 blocks
    // -- spreading its loads, stores and SiLU over more CUs.
    p.tpt_apply = 4;
    if ((tokens + p.rows * 4 - 1) / (p.rows * 4) < 256)
        p.tpt_apply = (tokens + p.rows * 2 - 1) / (p.rows * 2) >= 128 ? 2 : 1;
    p.tok_per_blk_apply = p.rows * p.tpt_apply;
    p.nblk_apply = (int)((tokens + p.tok_per_blk_apply - 1) / p.tok_per_blk_apply);
    // Statistics split (depends only on the geometry).  Up to nb_max blocks per batch: at most
    // 256, at most what a normalising block sums in one round of loads (16 in flight on each of
    // its threads / G lanes per group), and few enough that the partials all normalising blocks
    // read stay near 64 Ki (blocks x partials) -- a small band spreads over the whole GPU, a
    // large one keeps its partials few.  Each block takes its tokens in rows of R (token rows
    // r, r+R, ...), R the fewest (at most the normalising block's rows) that keep every thread
    // to one round of 8 loads; past that, whole rounds.
    int nb_max = 16 * (p.threads / G);
    if (nb_max > 256) nb_max = 256;
    int nb_vol = (int)(65536 / (p.nblk_apply > 0 ? p.nblk_apply : 1));
    if (nb_vol < 64) nb_vol = 64;
    if (nb_max > nb_vol) nb_max = nb_vol;
    const int64_t tpb0 = (tokens + nb_max - 1) / nb_max;           // tokens per block
    int64_t rs = (tpb0 + 7) / 8;
    if (rs > p.rows) rs = p.rows;
    if (rs < 1) rs = 1;
    p.rows_stats = (int)rs;
    p.threads_stats = p.vpt * p.rows_stats;
    int64_t tpb = (tpb0 + rs - 1) / rs * rs;
    if (tpb > 8 * rs) tpb = (tpb0 + 8 * rs - 1) / (8 * rs) * (8 * rs);   // whole rounds
    p.tok_per_blk = (int)tpb;
    p.nblk = (int)((tokens + tpb - 1) / tpb);
    p.partial_floats = (size_t)p.nblk * g.B * G * 2;
    p.ws_bytes = p.partial_floats * sizeof(float);
    return p;
}

hipError_t launch_gn_stats(const Geom& g, const GnPlan& plan, bool bf16, int G, const void* x, void* ws,
                           hipStream_t stream) {
    const dim3 grid((unsigned)plan.nblk, (unsigned)g.B);
    const size_t shmem = gn_stats_lds_bytes(g, plan);
    if (bf16)
        gn_stats_kernel<true><<<grid, plan.threads_stats, shmem, stream>>>(x, g.band_tokens(), g.C, G, plan.vpt,
                                                                          plan.rows_stats, plan.tok_per_blk,
                                                                          (float2*)ws);
    else
        gn_stats_kernel<false><<<grid, plan.threads_stats, shmem, stream>>>(x, g.band_tokens(), g.C, G, plan.vpt,
                                                                           plan.rows_stats, plan.tok_per_blk,
                                                                           (float2*)ws);
    return hipGetLastError();
}

float gn_inv_count(const Geom& g, int G) { return 1.0f / (float)((double)g.band_tokens() * (g.C / G)); }

hipError_t launch_groupnorm(const Geom& g, const GnPlan& plan, bool bf16, int G, float eps, int mode, int act,
                            const void* x, const float* stale_stats, const float* gamma, const float* beta,
                            float* fresh_stats_out, void* y, void* ws, hipStream_t stream) {
    GnApplyArgs a;
    a.x = x;
    a.y = y;
    a.partial = (const float2*)ws;
    a.nblk = plan.nblk;
    a.tokens = g.band_tokens();
    a.B = g.B;
    a.C = g.C;
    a.G = G;
    a.P = g.P;
    a.i = g.i;
    a.mode = y ? mode : 1;   // moments only: the table is not read
    a.vpt = plan.vpt;
    a.rows = plan.rows;
    a.tok_per_blk = 0;
    a.inv_count = gn_inv_count(g, G);
    a.eps = eps;
    a.stale = stale_stats;
    a.gamma = gamma;
    a.beta = beta;
    a.fresh_out = fresh_stats_out;
    float2* partial = (float2*)ws;
    if (bf16) return act == 1 ? launch_gn_typed<true, true>(g, plan, a, partial, stream)
                              : launch_gn_typed<true, false>(g, plan, a, partial, stream);
    return act == 1 ? launch_gn_typed<false, true>(g, plan, a, partial, stream)
                    : launch_gn_typed<false, false>(g, plan, a, partial, stream);
}

}  // namespace dp
