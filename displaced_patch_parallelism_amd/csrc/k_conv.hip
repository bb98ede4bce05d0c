// 3x3 convolution of one patch with stale halo rows.
//
// Activation displacement (study.space page, Method): a patch computes only
// its own rows, and the context it needs from neighbouring patches -- for a
// 3x3 conv, the row just above and the row just below its band -- is taken
// from the previous step's map.  The conv is the zero-padded, stride-1 3x3
// cross-correlation of the spliced map evaluated on the band:
//   y[b,y,x,o] = bias[o] + sum_{ky,kx,c} w[o,ky,kx,c] * src(b, r0+y+ky-1, x+kx-1, c)
// src = fresh patch inside the band, stale map at other image rows, 0 outside.
//
// bf16 path: implicit GEMM on MFMA (v_mfma_f32_32x32x16_bf16).
//   M = B*h*W output pixels, N = Cout, K = 9*Cin with k = tap*Cin + c, so a
//   K tile of 64 lies inside one tap.  Weights [Cout][3][3][Cin] are the GEMM's
//   B^T, row-contiguous in K.  The A loader resolves each pixel's source row
//   once per tap (fresh band / stale map / zero) and then streams 128-byte
//   channel runs; rows are staged through LDS with a 16-byte pad per row.
//   Tile 128 pixels x 160 channels, 4 waves, each wave 32 pixels x 160
//   channels (5 MFMA blocks).  Small M is split along K; the fp32 partials
//   are summed in split order by a second kernel (deterministic).
// f32 path: one thread per output element (correctness path for small maps).

#include "dp_device.h"
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int BM = 128;
constexpr int BN = 160;
constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
constexpr int NB = BN / 32;  // MFMA n-blocks per wave
constexpr int kThreads = 256;

struct ConvArgs {
    const uint16_t* xp;
    const uint16_t* xs;
    const uint16_t* w;
    const float* bias;
    uint16_t* y;
    float* part;
    int B, H, W, Cin, Cout, h, r0;
    int M;
    int ktiles, ksplit;
    int ntiles;
};

__global__ __launch_bounds__(kThreads) void conv3x3_bf16_mfma_kernel(ConvArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mt = blockIdx.x / a.ntiles;
    const int nt = blockIdx.x % a.ntiles;
    const int m0 = mt * BM;
    const int n0 = nt * BN;
    const int split = blockIdx.y;
    const int kt0 = (int)((int64_t)a.ktiles * split / a.ksplit);
    const int kt1 = (int)((int64_t)a.ktiles * (split + 1) / a.ksplit);
    const int cpt = a.Cin / BK;  // K tiles per tap

    // ---- per-thread loader state ----
    const int chunk = tid & 7;   // 16-byte chunk within a 128-byte K row
    const int lrow = tid >> 3;   // 0..31
    int pb[4], py[4], px[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + lrow + 32 * j;
        if (m < a.M) {
            const int hw = a.h * a.W;
            pb[j] = m / hw;
            const int rem = m - pb[j] * hw;
            py[j] = rem / a.W;
            px[j] = rem - py[j] * a.W;
        } else {
            pb[j] = -1;
            py[j] = px[j] = 0;
        }
    }
    const uint16_t* asrc[4];
    bool aval[4];
    int cur_tap = -1;

    auto set_tap = [&](int tap) {
        const int ky = tap / 3, kx = tap - 3 * (tap / 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = a.r0 + py[j] + ky - 1;
            const int xx = px[j] + kx - 1;
            aval[j] = pb[j] >= 0 && r >= 0 && r < a.H && xx >= 0 && xx < a.W;
            const bool fresh = r >= a.r0 && r < a.r0 + a.h;
            const int64_t fo = (((int64_t)pb[j] * a.h + (r - a.r0)) * a.W + xx) * a.Cin;
            const int64_t so = (((int64_t)pb[j] * a.H + r) * a.W + xx) * a.Cin;
            asrc[j] = aval[j] ? (fresh ? a.xp + fo : a.xs + so) : a.xp;
        }
    };

    uint4 ra[4], rb[NB];
    auto load_tile = [&](int kt) {
        const int tap = kt / cpt;
        const int c0 = (kt - tap * cpt) * BK + chunk * 8;
        if (tap != cur_tap) {
            set_tap(tap);
            cur_tap = tap;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ra[j] = aval[j] ? *(const uint4*)(asrc[j] + c0) : make_uint4(0, 0, 0, 0);
        const int64_t kofs = (int64_t)kt * BK + chunk * 8;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int co = n0 + lrow + 32 * j;
            rb[j] = co < a.Cout ? *(const uint4*)(a.w + (int64_t)co * 9 * a.Cin + kofs) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) *(uint4*)(As + (lrow + 32 * j) * LDK + chunk * 8) = ra[j];
#pragma unroll
        for (int j = 0; j < NB; ++j) *(uint4*)(Bs + (lrow + 32 * j) * LDK + chunk * 8) = rb[j];
    };

    f32x16 acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[n][e] = 0.f;

    if (kt0 < kt1) {
        load_tile(kt0);
        store_tile();
        __syncthreads();
    }
    const int arow = wave * 32 + (lane & 31);
    const int kl = (lane >> 5) * 8;
    for (int kt = kt0; kt < kt1; ++kt) {
        const bool more = kt + 1 < kt1;
        if (more) load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const bf16x8 af = *(const bf16x8*)(As + arow * LDK + ks * 16 + kl);
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const bf16x8 bfr = *(const bf16x8*)(Bs + (n * 32 + (lane & 31)) * LDK + ks * 16 + kl);
                acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[n], 0, 0, 0);
            }
        }
        __syncthreads();
        if (more) {
            store_tile();
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds column (l & 31) of each n-block, rows 8q + 4(l>>5) + r ----
    const int col = lane & 31;
    const int rbase = wave * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int co = n0 + n * 32 + col;
        if (co >= a.Cout) continue;
        const float bv = (a.ksplit == 1 && a.bias) ? a.bias[co] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + rbase + 8 * q + r;
                if (m >= a.M) continue;
                const float v = acc[n][4 * q + r];
                if (a.ksplit == 1)
                    a.y[(int64_t)m * a.Cout + co] = f32_to_bf16(v + bv);
                else
                    a.part[((int64_t)split * a.M + m) * a.Cout + co] = v;
            }
    }
}

// y[m][co] = bf16(bias[co] + sum_s part[s][m][co]), summed in split order.
__global__ __launch_bounds__(256) void conv_splitk_reduce_kernel(const float* __restrict__ part,
                                                                 const float* __restrict__ bias,
                                                                 uint16_t* __restrict__ y, int64_t total4,
                                                                 int Cout, int ksplit) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i4 >= total4) return;
    const int64_t i = i4 * 4;
    float4 s = *(const float4*)(part + i);
    for (int k = 1; k < ksplit; ++k) {
        const float4 v = *(const float4*)(part + (int64_t)k * total4 * 4 + i);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const int co = (int)(i % Cout);
    if (bias) {
        s.x += bias[co];
        s.y += bias[co + 1];
        s.z += bias[co + 2];
        s.w += bias[co + 3];
    }
    uint2 o;
    o.x = pack_bf16x2(s.x, s.y);
    o.y = pack_bf16x2(s.z, s.w);
    *(uint2*)(y + i) = o;
}

__global__ __launch_bounds__(256) void conv3x3_f32_direct_kernel(const float* __restrict__ xp,
                                                                 const float* __restrict__ xs,
                                                                 const float* __restrict__ w,
                                                                 const float* __restrict__ bias,
                                                                 float* __restrict__ y, int B, int H, int W,
                                                                 int Cin, int Cout, int h, int r0) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)B * h * W * Cout;
    if (idx >= total) return;
    const int o = (int)(idx % Cout);
    const int64_t pix = idx / Cout;
    const int x = (int)(pix % W);
    const int yy = (int)((pix / W) % h);
    const int b = (int)(pix / ((int64_t)W * h));
    float acc = bias ? bias[o] : 0.f;
    for (int ky = 0; ky < 3; ++ky) {
        const int r = r0 + yy + ky - 1;
        if (r < 0 || r >= H) continue;
        for (int kx = 0; kx < 3; ++kx) {
            const int xx = x + kx - 1;
            if (xx < 0 || xx >= W) continue;
            const float* src = (r >= r0 && r < r0 + h) ? xp + (((int64_t)b * h + (r - r0)) * W + xx) * Cin
                                                       : xs + (((int64_t)b * H + r) * W + xx) * Cin;
            const float* wp = w + (((int64_t)o * 3 + ky) * 3 + kx) * Cin;
            for (int c = 0; c < Cin; ++c) acc = fmaf(wp[c], src[c], acc);
        }
    }
    y[idx] = acc;
}

}  // namespace

ConvPlan plan_conv(const Geom& g, int Cout, bool bf16) {
    ConvPlan p{};
    if (!bf16) {
        p.kind = 0;
        return p;
    }
    p.kind = 1;
    p.bm = BM;
    p.bn = BN;
    const int64_t M = (int64_t)g.B * g.h * g.W;
    p.mtiles = (int)((M + BM - 1) / BM);
    p.ntiles = (Cout + BN - 1) / BN;
    p.ktiles = 9 * g.C / BK;
    const int tiles = p.mtiles * p.ntiles;
    int ks = 1;
    if (tiles < 256) {
        ks = (256 + tiles - 1) / tiles;
        const int maxk = p.ktiles / 4 > 0 ? p.ktiles / 4 : 1;  // keep >= 4 K tiles per split
        if (ks > maxk) ks = maxk;
        if (ks > 32) ks = 32;
    }
    p.ksplit = ks;
    p.ws_bytes = ks > 1 ? (size_t)ks * M * Cout * sizeof(float) : 0;
    return p;
}

hipError_t launch_conv(const Geom& g, const ConvPlan& plan, bool bf16, int Cout, const void* x_patch,
                       const void* x_stale, const void* w, const float* bias, void* y, void* ws,
                       hipStream_t stream) {
    if (!bf16) {
        const int64_t total = (int64_t)g.B * g.h * g.W * Cout;
        const int64_t blocks = (total + 255) / 256;
        conv3x3_f32_direct_kernel<<<(unsigned)blocks, 256, 0, stream>>>(
            (const float*)x_patch, (const float*)x_stale, (const float*)w, bias, (float*)y, g.B, g.H, g.W, g.C, Cout,
            g.h, g.r0);
        return hipGetLastError();
    }
    ConvArgs a;
    a.xp = (const uint16_t*)x_patch;
    a.xs = (const uint16_t*)x_stale;
    a.w = (const uint16_t*)w;
    a.bias = bias;
    a.y = (uint16_t*)y;
    a.part = (float*)ws;
    a.B = g.B;
    a.H = g.H;
    a.W = g.W;
    a.Cin = g.C;
    a.Cout = Cout;
    a.h = g.h;
    a.r0 = g.r0;
    a.M = g.B * g.h * g.W;
    a.ktiles = plan.ktiles;
    a.ksplit = plan.ksplit;
    a.ntiles = plan.ntiles;
    dim3 grid((unsigned)(plan.mtiles * plan.ntiles), (unsigned)plan.ksplit);
    conv3x3_bf16_mfma_kernel<<<grid, kThreads, 0, stream>>>(a);
    if (plan.ksplit > 1) {
        const int64_t total4 = (int64_t)a.M * Cout / 4;
        conv_splitk_reduce_kernel<<<(unsigned)((total4 + 255) / 256), 256, 0, stream>>>(
            (const float*)ws, bias, (uint16_t*)y, total4, Cout, plan.ksplit);
    }
    return hipGetLastError();
}

}  // namespace dp
