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
// Three launches, all streaming over the band [B][h*W][C] with 16-byte
// vectors:
//   1. gn_stats:    each block owns a token range; thread (cv, r) owns
//                   channel vector cv and walks tokens r, r+R, ...; fp32
//                   per-channel sums, reduced through LDS in a fixed order to
//                   per-group partial (sum, sum of squares) per block.
//   2. gn_finalize: one wave per (b, g) adds the block partials in a fixed
//                   order, emits (m_i, q_i), combines with the stale table
//                   and stores (mean, rstd).
//   3. gn_apply:    y = x * a[c] + b'[c] with a = rstd*gamma,
//                   b' = beta - mean*a, optional SiLU, rounded to the
//                   storage type.
// No atomics: results are bitwise reproducible.

#include "dp_device.h"
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kApplyThreads = 256;
constexpr int kApplyUnroll = 4;

template <bool BF16>
__device__ __forceinline__ void load_vec(const void* base, int64_t vec_index, float* f) {
    const uint4 v = ((const uint4*)base)[vec_index];
    if (BF16) {
        unpack8(v, f);
    } else {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
}

// partial[(b*nblk + blk)*G + g] = (sum x, sum x^2) over the block's tokens.
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
    const int64_t batch_vec0 = (int64_t)b * tokens * vpt;
    for (int64_t t = t0 + r; t < t1; t += rows) {
        float f[VEC];
        load_vec<BF16>(x, batch_vec0 + t * vpt + cv, f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            s[e] += f[e];
            q[e] = fmaf(f[e], f[e], q[e]);
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
    // per-channel totals over the rows, in row order; kept in row 0
    for (int c = tid; c < C; c += blockDim.x) {
        float a = sh_s[c], aq = sh_q[c];
        for (int j = 1; j < rows; ++j) {
            a += sh_s[j * C + c];
            aq += sh_q[j * C + c];
        }
        sh_s[c] = a;
        sh_q[c] = aq;
    }
    __syncthreads();
    const int cg = C / G;
    for (int g = tid; g < G; g += blockDim.x) {
        float a = 0.f, aq = 0.f;
        for (int c = g * cg; c < (g + 1) * cg; ++c) {
            a += sh_s[c];
            aq += sh_q[c];
        }
        partial[((int64_t)b * gridDim.x + blockIdx.x) * G + g] = make_float2(a, aq);
    }
}

// One wave per (b, g).  meanrstd[b*G + g] = (mean, rstd).
__global__ __launch_bounds__(256) void gn_finalize_kernel(const float2* __restrict__ partial, int nblk, int B,
                                                          int G, int P, int i, int mode, float inv_count,
                                                          float eps, const float* __restrict__ stale,
                                                          float* __restrict__ fresh_out,
                                                          float2* __restrict__ meanrstd, int need_norm) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (wave >= B * G) return;
    const int b = wave / G, g = wave % G;
    float a = 0.f, aq = 0.f;
    for (int j = lane; j < nblk; j += 64) {
        const float2 v = partial[((int64_t)b * nblk + j) * G + g];
        a += v.x;
        aq += v.y;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        a += __shfl_xor(a, off);
        aq += __shfl_xor(aq, off);
    }
    if (lane != 0) return;
    const float m = a * inv_count, qm = aq * inv_count;
    if (fresh_out) {
        fresh_out[(b * G + g) * 2 + 0] = m;
        fresh_out[(b * G + g) * 2 + 1] = qm;
    }
    if (!need_norm) return;
    float E = m, Q = qm;
    if (mode != 1) {  // corrected (0) or stale (2): sum the table in band order
        float se = 0.f, sq = 0.f;
        for (int j = 0; j < P; ++j) {
            if (mode == 0 && j == i) {
                se += m;
                sq += qm;
            } else {
                se += stale[((int64_t)j * B + b) * G * 2 + g * 2 + 0];
                sq += stale[((int64_t)j * B + b) * G * 2 + g * 2 + 1];
            }
        }
        E = se / (float)P;
        Q = sq / (float)P;
    }
    const float var = fmaxf(Q - E * E, 0.f);
    meanrstd[b * G + g] = make_float2(E, 1.0f / sqrtf(var + eps));
}

template <bool BF16, bool SILU>
__global__ __launch_bounds__(kApplyThreads) void gn_apply_kernel(const void* __restrict__ x, void* __restrict__ y,
                                                                 int64_t nvec, int vpt, int C, int G,
                                                                 const float2* __restrict__ meanrstd,
                                                                 const float* __restrict__ gamma,
                                                                 const float* __restrict__ beta) {
    constexpr int VEC = BF16 ? 8 : 4;
    extern __shared__ float2 ab[];  // [C] (scale, shift)
    const int b = blockIdx.y;
    const int cg = C / G;
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
        const float2 mr = meanrstd[b * G + c / cg];
        const float ga = gamma ? gamma[c] : 1.f;
        const float be = beta ? beta[c] : 0.f;
        const float sc = mr.y * ga;
        ab[c] = make_float2(sc, be - mr.x * sc);
    }
    __syncthreads();
    const int64_t batch0 = (int64_t)b * nvec;
    const int64_t stride = (int64_t)gridDim.x * kApplyThreads * kApplyUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kApplyThreads * kApplyUnroll + threadIdx.x; base < nvec;
         base += stride) {
        uint4 raw[kApplyUnroll];
#pragma unroll
        for (int u = 0; u < kApplyUnroll; ++u) {
            const int64_t v = base + u * kApplyThreads;
            if (v < nvec) raw[u] = ((const uint4*)x)[batch0 + v];
        }
#pragma unroll
        for (int u = 0; u < kApplyUnroll; ++u) {
            const int64_t v = base + u * kApplyThreads;
            if (v >= nvec) continue;
            const int c0 = (int)(v % vpt) * VEC;
            float f[VEC];
            if (BF16) {
                unpack8(raw[u], f);
            } else {
                f[0] = __uint_as_float(raw[u].x);
                f[1] = __uint_as_float(raw[u].y);
                f[2] = __uint_as_float(raw[u].z);
                f[3] = __uint_as_float(raw[u].w);
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float2 k = ab[c0 + e];
                float t = fmaf(f[e], k.x, k.y);
                if (SILU) t = silu(t);
                f[e] = t;
            }
            uint4 out;
            if (BF16) {
                out = pack8(f);
            } else {
                out = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                                 __float_as_uint(f[3]));
            }
            ((uint4*)y)[batch0 + v] = out;
        }
    }
}

}  // namespace

GnPlan plan_groupnorm(const Geom& g, int G, bool bf16) {
    GnPlan p{};
    p.vec = bf16 ? 8 : 4;
    p.vpt = g.C / p.vec;
    p.rows = p.vpt >= 512 ? 1 : 512 / p.vpt;
    p.threads = p.vpt * p.rows;
    const int64_t tokens = g.band_tokens();
    // about 512 blocks over the whole band, at least ~2 token rows per thread row
    int64_t want = 512 / g.B;
    if (want < 1) want = 1;
    int64_t per = (tokens + want - 1) / want;
    const int64_t min_per = 2 * (int64_t)p.rows;
    if (per < min_per) per = min_per;
    p.tok_per_blk = (int)per;
    p.nblk = (int)((tokens + per - 1) / per);
    if (p.nblk < 1) p.nblk = 1;
    p.partial_floats = (size_t)g.B * p.nblk * G * 2;
    const size_t partial_bytes = (p.partial_floats * sizeof(float) + 255) & ~(size_t)255;
    p.ws_bytes = partial_bytes + (size_t)g.B * G * 2 * sizeof(float);
    return p;
}

hipError_t launch_groupnorm(const Geom& g, const GnPlan& plan, bool bf16, int G, float eps, int mode, int act,
                            const void* x, const float* stale_stats, const float* gamma, const float* beta,
                            float* fresh_stats_out, void* y, void* ws, hipStream_t stream) {
    float2* partial = (float2*)ws;
    const size_t partial_bytes = (plan.partial_floats * sizeof(float) + 255) & ~(size_t)255;
    float2* meanrstd = (float2*)((char*)ws + partial_bytes);
    const int64_t tokens = g.band_tokens();
    {
        dim3 grid((unsigned)plan.nblk, (unsigned)g.B);
        const size_t shmem = (size_t)2 * plan.rows * g.C * sizeof(float);
        if (bf16)
            gn_stats_kernel<true><<<grid, plan.threads, shmem, stream>>>(x, tokens, g.C, G, plan.vpt, plan.rows,
                                                                        plan.tok_per_blk, partial);
        else
            gn_stats_kernel<false><<<grid, plan.threads, shmem, stream>>>(x, tokens, g.C, G, plan.vpt, plan.rows,
                                                                         plan.tok_per_blk, partial);
    }
    {
        const int waves = g.B * G;
        const int blocks = (waves * 64 + 255) / 256;
        const float inv_count = 1.0f / (float)((double)tokens * (g.C / G));
        gn_finalize_kernel<<<blocks, 256, 0, stream>>>(partial, plan.nblk, g.B, G, g.P, g.i, mode, inv_count, eps,
                                                       stale_stats, fresh_stats_out, meanrstd, y != nullptr);
    }
    if (y) {
        const int64_t nvec = tokens * plan.vpt;
        int64_t blocks = (nvec + kApplyThreads * kApplyUnroll - 1) / (kApplyThreads * kApplyUnroll);
        if (blocks > 2048) blocks = 2048;
        dim3 grid((unsigned)blocks, (unsigned)g.B);
        const size_t shmem = (size_t)g.C * sizeof(float2);
        const bool silu_on = act == 1;
        if (bf16) {
            if (silu_on)
                gn_apply_kernel<true, true><<<grid, kApplyThreads, shmem, stream>>>(x, y, nvec, plan.vpt, g.C, G,
                                                                                   meanrstd, gamma, beta);
            else
                gn_apply_kernel<true, false><<<grid, kApplyThreads, shmem, stream>>>(x, y, nvec, plan.vpt, g.C, G,
                                                                                    meanrstd, gamma, beta);
        } else {
            if (silu_on)
                gn_apply_kernel<false, true><<<grid, kApplyThreads, shmem, stream>>>(x, y, nvec, plan.vpt, g.C, G,
                                                                                    meanrstd, gamma, beta);
            else
                gn_apply_kernel<false, false><<<grid, kApplyThreads, shmem, stream>>>(x, y, nvec, plan.vpt, g.C,
                                                                                     G, meanrstd, gamma, beta);
        }
    }
    return hipGetLastError();
}

}  // namespace dp
