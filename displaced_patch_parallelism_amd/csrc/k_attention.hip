// Self-attention of one patch over the stale K/V with the fresh patch spliced in.
//
// DistriFusion keeps the full spatial K and V of every layer on every device
// (PipeFusion explainer on gist.science, Problem Statement and Memory
// Efficiency); a patch's queries attend to all H*W tokens, its own band
// being fresh (activation displacement, study.space page, Method).  For head
// e (channels [e*d, (e+1)*d)):
//   O[q] = sum_n softmax_n(scale * <Q[q], K[n]>) V[n],
//   K[n] = k_patch[n - r0*W] for n in the band, k_stale[n] elsewhere (same for V).
//
// bf16 path (d = 64): flash-style single pass with an online softmax in the
// base-2 domain (log2(e) folded into the scale).  A workgroup holds 128
// queries (4 waves x 32); K/V tiles of 64 tokens are staged in LDS, K
// row-major and V transposed.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so that lane l owns query l%32: the running max
// and sum stay in the lane (one cross-half exchange per tile for the max).
// P^T (bf16) feeds O^T = V^T P^T directly from registers; within each 16-key
// MFMA step the key order is permuted identically on both operands so the
// S^T accumulator layout needs no shuffle.  The token loader picks the fresh
// or stale buffer per key row, so tiles may straddle the band edges.  When
// (query tiles x heads) cannot fill the GPU, keys are split and the partial
// (O, max, sum) are merged by a second kernel in split order.
// f32 path: one thread per (query, head), online softmax, for small maps.

#include "dp_device.h"
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int D = 64;
constexpr int QT = 128;         // queries per workgroup
constexpr int KT = 64;          // keys per tile
constexpr int LDKS = D + 8;     // K tile row stride (bf16)
constexpr int LDVT = KT + 8;    // V^T tile row stride (bf16)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* ks;
    const uint16_t* vs;
    uint16_t* o;
    float* part_o;     // [split][B*heads][Nq][D]
    float2* part_ml;   // [split][B*heads][Nq] (max, sum)
    int B, heads, C, Nq, N, band0;
    int kv_tiles, kvsplit;
    float sc;          // scale * log2(e)
};

__device__ __forceinline__ const uint16_t* kv_row(const uint16_t* fresh, const uint16_t* stale, int b, int n,
                                                  const AttnArgs& a, int col) {
    const int rel = n - a.band0;
    if (rel >= 0 && rel < a.Nq) return fresh + ((int64_t)b * a.Nq + rel) * a.C + col;
    return stale + ((int64_t)b * a.N + n) * a.C + col;
}

template <int QA>
__device__ __forceinline__ bf16x8 pack_probs(const f32x16& p) {
    // keys 8*QA + {0..3} and 8*(QA+1) + {0..3} of the block (see the key permutation above)
    uint4 raw;
    raw.x = pack_bf16x2(p[4 * QA + 0], p[4 * QA + 1]);
    raw.y = pack_bf16x2(p[4 * QA + 2], p[4 * QA + 3]);
    raw.z = pack_bf16x2(p[4 * QA + 4], p[4 * QA + 5]);
    raw.w = pack_bf16x2(p[4 * QA + 6], p[4 * QA + 7]);
    return __builtin_bit_cast(bf16x8, raw);
}

__device__ __forceinline__ bf16x8 load_vt(const uint16_t* vrow) {
    const uint2 lo = *(const uint2*)vrow;
    const uint2 hi = *(const uint2*)(vrow + 8);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

__device__ __forceinline__ void stage_kv(uint16_t* Ks, uint16_t* Vt, int kr, int chunk, const uint4& k4,
                                         const uint4& v4) {
    *(uint4*)(Ks + kr * LDKS + chunk * 8) = k4;
    uint16_t* vt = Vt + chunk * 8 * LDVT + kr;
    vt[0 * LDVT] = (uint16_t)(v4.x & 0xffffu);
    vt[1 * LDVT] = (uint16_t)(v4.x >> 16);
    vt[2 * LDVT] = (uint16_t)(v4.y & 0xffffu);
    vt[3 * LDVT] = (uint16_t)(v4.y >> 16);
    vt[4 * LDVT] = (uint16_t)(v4.z & 0xffffu);
    vt[5 * LDVT] = (uint16_t)(v4.z >> 16);
    vt[6 * LDVT] = (uint16_t)(v4.w & 0xffffu);
    vt[7 * LDVT] = (uint16_t)(v4.w >> 16);
}

__device__ __forceinline__ void fetch_kv(const AttnArgs& a, int b, int n, int col, uint4& k4, uint4& v4) {
    if (n < a.N) {
        k4 = *(const uint4*)kv_row(a.k, a.ks, b, n, a, col);
        v4 = *(const uint4*)kv_row(a.v, a.vs, b, n, a, col);
    } else {
        k4 = v4 = make_uint4(0, 0, 0, 0);
    }
}

__global__ __launch_bounds__(kThreads) void attn_bf16_d64_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * LDKS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LDVT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hsel = lane >> 5;          // which half of the wave
    const int bh = blockIdx.y;
    const int b = bh / a.heads;
    const int e = bh - b * a.heads;
    const int split = blockIdx.z;
    const int myq = blockIdx.x * QT + wave * 32 + (lane & 31);
    const bool qvalid = myq < a.Nq;
    const int col0 = e * D;

    // Q^T fragments (B operand): lane gives query myq, dims ks*16 + 8*hsel .. +7
    bf16x8 q0, q1, q2, q3;
    {
        uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0, r2 = r0, r3 = r0;
        if (qvalid) {
            const uint16_t* qp = a.q + ((int64_t)b * a.Nq + myq) * a.C + col0 + hsel * 8;
            r0 = *(const uint4*)(qp + 0);
            r1 = *(const uint4*)(qp + 16);
            r2 = *(const uint4*)(qp + 32);
            r3 = *(const uint4*)(qp + 48);
        }
        q0 = __builtin_bit_cast(bf16x8, r0);
        q1 = __builtin_bit_cast(bf16x8, r1);
        q2 = __builtin_bit_cast(bf16x8, r2);
        q3 = __builtin_bit_cast(bf16x8, r3);
    }

    const int t0 = (int)((int64_t)a.kv_tiles * split / a.kvsplit);
    const int t1 = (int)((int64_t)a.kv_tiles * (split + 1) / a.kvsplit);

    // loader: thread -> key rows lrow, lrow+32; 16-byte chunk `chunk` of the 128-byte head slice
    const int chunk = tid & 7;
    const int lrow = tid >> 3;
    const int lcol = col0 + chunk * 8;
    uint4 k4a, v4a, k4b, v4b;

    f32x16 o0, o1;
#pragma unroll
    for (int i = 0; i < 16; ++i) o0[i] = o1[i] = 0.f;
    float m_run = kNegBig;
    float l_run = 0.f;

    if (t0 < t1) {
        fetch_kv(a, b, t0 * KT + lrow, lcol, k4a, v4a);
        fetch_kv(a, b, t0 * KT + lrow + 32, lcol, k4b, v4b);
        stage_kv(Ks, Vt, lrow, chunk, k4a, v4a);
        stage_kv(Ks, Vt, lrow + 32, chunk, k4b, v4b);
        __syncthreads();
    }
    const uint16_t* krow0 = Ks + (lane & 31) * LDKS + hsel * 8;
    const uint16_t* krow1 = krow0 + 32 * LDKS;
    const uint16_t* vrow0 = Vt + (lane & 31) * LDVT + 4 * hsel;
    const uint16_t* vrow1 = vrow0 + 32 * LDVT;
    for (int t = t0; t < t1; ++t) {
        const bool more = t + 1 < t1;
        if (more) {
            fetch_kv(a, b, (t + 1) * KT + lrow, lcol, k4a, v4a);
            fetch_kv(a, b, (t + 1) * KT + lrow + 32, lcol, k4b, v4b);
        }
        // S^T[key][query], keys kb*32 + 8q + 4*hsel + r in s_kb[4q + r]
        f32x16 s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow0 + 0), q0, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow1 + 0), q0, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow0 + 16), q1, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow1 + 16), q1, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow0 + 32), q2, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow1 + 32), q2, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow0 + 48), q3, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(krow1 + 48), q3, s1, 0, 0, 0);

        // keys >= N (ragged last tile) are excluded from the max and get p = 0
        const int kvalid = a.N - (t * KT + 4 * hsel);  // element at block offset off is valid iff off < kvalid
        float mx = kNegBig;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int off = 8 * (i >> 2) + (i & 3);
            mx = fmaxf(mx, off < kvalid ? s0[i] : kNegBig);
            mx = fmaxf(mx, off + 32 < kvalid ? s1[i] : kNegBig);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * a.sc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int off = 8 * (i >> 2) + (i & 3);
            const float p0 = off < kvalid ? __builtin_amdgcn_exp2f(fmaf(s0[i], a.sc, -m_new)) : 0.f;
            const float p1 = off + 32 < kvalid ? __builtin_amdgcn_exp2f(fmaf(s1[i], a.sc, -m_new)) : 0.f;
            psum += p0 + p1;
            s0[i] = p0;
            s1[i] = p1;
        }
        l_run = fmaf(l_run, alpha, psum);
        o0 *= alpha;
        o1 *= alpha;
        // O^T[d][query] += V^T P^T over 4 steps of 16 keys (keys 16u + 4*hsel + {0..3, 8..11})
        const bf16x8 p0 = pack_probs<0>(s0);
        const bf16x8 p1 = pack_probs<2>(s0);
        const bf16x8 p2 = pack_probs<0>(s1);
        const bf16x8 p3 = pack_probs<2>(s1);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow0 + 0), p0, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow1 + 0), p0, o1, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow0 + 16), p1, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow1 + 16), p1, o1, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow0 + 32), p2, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow1 + 32), p2, o1, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow0 + 48), p3, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_vt(vrow1 + 48), p3, o1, 0, 0, 0);
        __syncthreads();
        if (more) {
            stage_kv(Ks, Vt, lrow, chunk, k4a, v4a);
            stage_kv(Ks, Vt, lrow + 32, chunk, k4b, v4b);
            __syncthreads();
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!qvalid) return;
    // O^T layout: lane owns query myq, dims db*32 + 8q + 4*hsel + r
    if (a.kvsplit == 1) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = a.o + ((int64_t)b * a.Nq + myq) * a.C + col0 + 4 * hsel;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint2 w;
            w.x = pack_bf16x2(o0[4 * q + 0] * inv, o0[4 * q + 1] * inv);
            w.y = pack_bf16x2(o0[4 * q + 2] * inv, o0[4 * q + 3] * inv);
            *(uint2*)(orow + 8 * q) = w;
            w.x = pack_bf16x2(o1[4 * q + 0] * inv, o1[4 * q + 1] * inv);
            w.y = pack_bf16x2(o1[4 * q + 2] * inv, o1[4 * q + 3] * inv);
            *(uint2*)(orow + 32 + 8 * q) = w;
        }
    } else {
        const int64_t row = ((int64_t)split * a.B * a.heads + bh) * a.Nq + myq;
        float* prow = a.part_o + row * D + 4 * hsel;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *(float4*)(prow + 8 * q) = make_float4(o0[4 * q + 0], o0[4 * q + 1], o0[4 * q + 2], o0[4 * q + 3]);
            *(float4*)(prow + 32 + 8 * q) = make_float4(o1[4 * q + 0], o1[4 * q + 1], o1[4 * q + 2], o1[4 * q + 3]);
        }
        if (hsel == 0) a.part_ml[row] = make_float2(m_run, l_tot);
    }
}

// Merge of key-split partials, in split order.  One thread per (b*heads, query, 4 dims).
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         uint16_t* __restrict__ o, int B, int heads, int C,
                                                         int Nq, int kvsplit) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)B * heads * Nq;
    if (idx >= rows * (D / 4)) return;
    const int d4 = (int)(idx % (D / 4));
    const int64_t row = idx / (D / 4);  // (bh, q)
    const int q = (int)(row % Nq);
    const int bh = (int)(row / Nq);
    float M = kNegBig;
    for (int s = 0; s < kvsplit; ++s) M = fmaxf(M, part_ml[(int64_t)s * rows + row].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < kvsplit; ++s) {
        const float2 ml = part_ml[(int64_t)s * rows + row];
        const float w = __builtin_amdgcn_exp2f(ml.x - M);
        L = fmaf(ml.y, w, L);
        const float4 v = *(const float4*)(part_o + ((int64_t)s * rows + row) * D + d4 * 4);
        acc.x = fmaf(v.x, w, acc.x);
        acc.y = fmaf(v.y, w, acc.y);
        acc.z = fmaf(v.z, w, acc.z);
        acc.w = fmaf(v.w, w, acc.w);
    }
    const float inv = 1.0f / L;
    const int b = bh / heads, e = bh - (bh / heads) * heads;
    uint2 w2;
    w2.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    w2.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *(uint2*)(o + ((int64_t)b * Nq + q) * C + e * D + d4 * 4) = w2;
}

template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, const float* __restrict__ ks,
                                                      const float* __restrict__ vs, float* __restrict__ o,
                                                      int B, int heads, int C, int Nq, int N, int band0,
                                                      float sc) {
    const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (idx >= (int64_t)B * heads * Nq) return;
    const int qi = (int)(idx % Nq);
    const int e = (int)((idx / Nq) % heads);
    const int b = (int)(idx / ((int64_t)Nq * heads));
    const int col = e * HD;
    float qv[HD], acc[HD];
    const float* qp = q + ((int64_t)b * Nq + qi) * C + col;
#pragma unroll
    for (int j = 0; j < HD; ++j) {
        qv[j] = qp[j];
        acc[j] = 0.f;
    }
    float m = kNegBig, l = 0.f;
    for (int n = 0; n < N; ++n) {
        const int rel = n - band0;
        const bool fresh = rel >= 0 && rel < Nq;
        const float* kp = fresh ? k + ((int64_t)b * Nq + rel) * C + col : ks + ((int64_t)b * N + n) * C + col;
        const float* vp = fresh ? v + ((int64_t)b * Nq + rel) * C + col : vs + ((int64_t)b * N + n) * C + col;
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < HD; ++j) dot = fmaf(qv[j], kp[j], dot);
        const float s = dot * sc;
        if (s > m) {
            const float alpha = exp2f(m - s);
            l *= alpha;
#pragma unroll
            for (int j = 0; j < HD; ++j) acc[j] *= alpha;
            m = s;
        }
        const float p = exp2f(s - m);
        l += p;
#pragma unroll
        for (int j = 0; j < HD; ++j) acc[j] = fmaf(p, vp[j], acc[j]);
    }
    float* op = o + ((int64_t)b * Nq + qi) * C + col;
    const float inv = 1.0f / l;
#pragma unroll
    for (int j = 0; j < HD; ++j) op[j] = acc[j] * inv;
}

}  // namespace

AttnPlan plan_attention(const Geom& g, int heads, int head_dim, bool bf16) {
    AttnPlan p{};
    if (!bf16) {
        p.kind = 0;
        p.kvsplit = 1;
        return p;
    }
    p.kind = 1;
    p.qtile = QT;
    const int64_t Nq = g.band_tokens();
    p.qtiles = (int)((Nq + QT - 1) / QT);
    const int kv_tiles = (int)((g.map_tokens() + KT - 1) / KT);
    const int64_t units = (int64_t)p.qtiles * g.B * heads;
    int ks = 1;
    while (units * ks * 2 <= 512 && kv_tiles / (ks * 2) >= 2) ks *= 2;
    p.kvsplit = ks;
    p.ws_bytes = ks > 1 ? (size_t)ks * g.B * heads * Nq * (D * sizeof(float) + sizeof(float2)) : 0;
    (void)head_dim;
    return p;
}

hipError_t launch_attention(const Geom& g, const AttnPlan& plan, bool bf16, int heads, int head_dim, float scale,
                            const void* q, const void* k, const void* v, const void* k_stale, const void* v_stale,
                            void* o, void* ws, hipStream_t stream) {
    const int Nq = (int)g.band_tokens();
    const int N = (int)g.map_tokens();
    const int band0 = g.r0 * g.W;
    if (!bf16) {
        const int64_t total = (int64_t)g.B * heads * Nq;
        const unsigned blocks = (unsigned)((total + 63) / 64);
        const float sc = scale * kLog2e;
#define DP_F32_ATTN(HD)                                                                                  \
    attn_f32_kernel<HD><<<blocks, 64, 0, stream>>>((const float*)q, (const float*)k, (const float*)v,   \
                                                   (const float*)k_stale, (const float*)v_stale,        \
                                                   (float*)o, g.B, heads, g.C, Nq, N, band0, sc)
        switch (head_dim) {
            case 4: DP_F32_ATTN(4); break;
            case 8: DP_F32_ATTN(8); break;
            case 16: DP_F32_ATTN(16); break;
            case 32: DP_F32_ATTN(32); break;
            case 64: DP_F32_ATTN(64); break;
            case 128: DP_F32_ATTN(128); break;
            default: return hipErrorInvalidValue;
        }
#undef DP_F32_ATTN
        return hipGetLastError();
    }
    AttnArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.ks = (const uint16_t*)k_stale;
    a.vs = (const uint16_t*)v_stale;
    a.o = (uint16_t*)o;
    const size_t po_bytes = (size_t)plan.kvsplit * g.B * heads * Nq * D * sizeof(float);
    a.part_o = (float*)ws;
    a.part_ml = (float2*)((char*)ws + po_bytes);
    a.B = g.B;
    a.heads = heads;
    a.C = g.C;
    a.Nq = Nq;
    a.N = N;
    a.band0 = band0;
    a.kv_tiles = (N + KT - 1) / KT;
    a.kvsplit = plan.kvsplit;
    a.sc = scale * kLog2e;
    dim3 grid((unsigned)plan.qtiles, (unsigned)(g.B * heads), (unsigned)plan.kvsplit);
    attn_bf16_d64_kernel<<<grid, kThreads, 0, stream>>>(a);
    if (plan.kvsplit > 1) {
        const int64_t threads = (int64_t)g.B * heads * Nq * (D / 4);
        attn_merge_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(
            a.part_o, a.part_ml, (uint16_t*)o, g.B, heads, g.C, Nq, plan.kvsplit);
    }
    return hipGetLastError();
}

}  // namespace dp
