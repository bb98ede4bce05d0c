// Learned projections of an attention layer: y = x W^T + bias.
//
// An attention layer with learned projections caches the projected K and V of
// the whole map (every device keeps the full spatial K/V of every layer:
// PipeFusion explainer on gist.science, Problem Statement and Memory
// Efficiency); a patch projects only its own tokens, writing its fresh K and V
// straight into band i of that cache, and projects the attention output by W_o.
//
// bf16 path: tiled GEMM on MFMA (v_mfma_f32_16x16x32_bf16).  Rows of x (tokens,
// row stride ldx) and of W (output channels) are both contiguous in K, so a K
// tile of 64 is one 128-byte line per row; tiles stream global -> LDS with
// direct-to-LDS loads (global_load_lds_dwordx4, lane l fills the l-th 16-byte
// slot of a 1 KB run; chunk c of row r at slot c ^ (r & 7)) through a 2-stage
// ring.  4 waves in a 2 x 2 grid; the output tile (acc + bias, fp32) is staged in
// LDS for coalesced 16-byte stores; an optional residual r (the skip connection
// of a transformer block's output projection) is added there before the single
// rounding to bf16.  Workgroups are renumbered so
// each XCD walks a contiguous run of row tiles (consecutive tiles share W).
// f32 path: one thread per output element.

#include "dp_device.h"
#include "dp_internal.h"

namespace dp {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __attribute__((aligned(64))) uint4 g_lin_zero[8];   // never written: a zero row

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct LinArgs {
    const uint16_t* x;
    const uint16_t* w;
    const float* bias;
    const uint16_t* r;       // residual [M][N] (row stride ldr) or null
    uint16_t* y;
    int64_t ldx, ldy, ldr;
    int M, N, K;
    int mtiles, ntiles;
    // segmented output (segw > 0): columns [s*segw, (s+1)*segw) of the product go to segment s
    // (y, y1, y2 with their row strides), column n - s*segw
    uint16_t* y1;
    uint16_t* y2;
    int64_t ldy1, ldy2;
    int segw;
};

template <int BM, int BN>
__global__ __launch_bounds__(256) void linear_bf16_kernel(LinArgs a) {
    constexpr int A_LOADS = BM / 8;              // 1 KB = 8 rows of 128 bytes
    constexpr int B_LOADS = BN / 8;
    constexpr int LOADS = A_LOADS + B_LOADS;
    static_assert(LOADS % 4 == 0, "loads dealt evenly to 4 waves");
    constexpr int LPW = LOADS / 4;
    constexpr int STAGE = LOADS * 1024;
    constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;     // 16x16 blocks per wave
    constexpr int TP = BN + 4;                    // fp32 output-tile pitch (padded: rows 4 apart
                                                  // would share banks)
    constexpr int SMEM = 2 * STAGE > BM * TP * 4 ? 2 * STAGE : BM * TP * 4;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, so each load's LDS destination is a scalar (no per-load readfirstlane)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    // XCD-contiguous order, row tile slowest: consecutive workgroups on an XCD share W
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int lt = xcd * (total >> 3) + (xcd < (total & 7) ? xcd : (total & 7)) + within;
    const int nt = lt % a.ntiles;
    const int mt = lt / a.ntiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const uint16_t* zero = (const uint16_t*)g_lin_zero;

    // this lane's rows of its loads: load q covers rows (q % (BM/8 or BN/8))*8 .. +7 of A or B
    const int sub = lane >> 3, slot = lane & 7;
    const uint16_t* src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int q = wave * LPW + j;
        if (q < A_LOADS) {
            const int r = q * 8 + sub;
            const int m = m0 + r;
            src[j] = m < a.M ? a.x + (int64_t)m * a.ldx + ((slot ^ (r & 7)) * 8) : nullptr;
        } else {
            const int r = (q - A_LOADS) * 8 + sub;
            int n = n0 + r;
            if (n >= a.N) n = a.N - 1;             // clamped rows feed columns never stored
            src[j] = a.w + (int64_t)n * a.K + ((slot ^ (r & 7)) * 8);
        }
    }
#define DPL_ISSUE(KT, BUF)                                                                          \
    do {                                                                                            \
        char* st_ = smem + (BUF) * STAGE;                                                           \
        _Pragma("unroll") for (int j = 0; j < LPW; ++j) {                                           \
            const uint16_t* g_ = src[j] ? src[j] + (KT) * 64 : zero;                                \
            __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + (wave * LPW + j) * 1024), \
                                             16, 0, 0);                                            \
        }                                                                                           \
    } while (0)

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int n = 0; n < FN; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand rows: A row wm*WM + 16i + (l & 15), B row BM + wn*WN + 16n + (l & 15); chunk
    // 4ks + (l >> 4) at slot chunk ^ (row & 7) (row & 7 = l & 7 since blocks start at multiples of 8)
    const int frow = lane & 15;
    const int po0 = ((0 + (lane >> 4)) ^ (lane & 7)) * 16;
    const int po1 = ((4 + (lane >> 4)) ^ (lane & 7)) * 16;
    const int aoff = (wm * WM + frow) * 128;
    const int boff = (BM + wn * WN + frow) * 128;

    const int nk = a.K / 64;
    DPL_ISSUE(0, 0);
    for (int it = 0; it < nk; ++it) {
        wait_vmcnt<0>();
        __syncthreads();
        if (it + 1 < nk) DPL_ISSUE(it + 1, (it + 1) & 1);
        const char* st = smem + (it & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int po = ks ? po1 : po0;
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8*)(st + aoff + i * 16 * 128 + po);
#pragma unroll
            for (int n = 0; n < FN; ++n) bfr[n] = *(const bf16x8*)(st + boff + n * 16 * 128 + po);
#pragma unroll
            for (int n = 0; n < FN; ++n)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], acc[i][n], 0, 0, 0);
        }
    }
#undef DPL_ISSUE
    __syncthreads();   // ring no longer read: reuse it for the output tile

    // acc[i][n][r] = D[row 16i + 4(l>>4) + r of the wave][column 16n + (l&15) of the wave]
    float* tile = (float*)smem;   // [BM][TP] fp32: acc + bias
    const int ecol = lane & 15, erow = 4 * (lane >> 4);
#pragma unroll
    for (int n = 0; n < FN; ++n) {
        const int c = wn * WN + n * 16 + ecol;
        const float bv = (a.bias && n0 + c < a.N) ? a.bias[n0 + c] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) tile[(wm * WM + i * 16 + erow + r) * TP + c] = acc[i][n][r] + bv;
    }
    __syncthreads();
    constexpr int CPR = BN / 8;   // 8-column (16-byte) output chunks per row
    for (int q = tid; q < BM * CPR; q += 256) {
        const int r = q / CPR, c8 = q - r * CPR;
        const int m = m0 + r, n = n0 + c8 * 8;
        if (m < a.M && n < a.N) {
            const float4 lo = *(const float4*)(tile + r * TP + c8 * 8);
            const float4 hi = *(const float4*)(tile + r * TP + c8 * 8 + 4);
            float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            if (a.r) {
                float rv[8];
                unpack8(*(const uint4*)(a.r + (int64_t)m * a.ldr + n), rv);
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] += rv[e];
            }
            uint16_t* yp = a.y;
            int64_t ld = a.ldy;
            int col = n;
            if (a.segw) {            // segments are multiples of 8 columns: a chunk lies in one
                const int sg = n / a.segw;
                col = n - sg * a.segw;
                if (sg == 1) {
                    yp = a.y1;
                    ld = a.ldy1;
                } else if (sg == 2) {
                    yp = a.y2;
                    ld = a.ldy2;
                }
            }
            *(uint4*)(yp + (int64_t)m * ld + col) = pack8(f);
        }
    }
}

__global__ __launch_bounds__(256) void linear_f32_kernel(const float* __restrict__ x, int64_t ldx,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ bias,
                                                         const float* __restrict__ r, int64_t ldr,
                                                         float* __restrict__ y, int64_t ldy, int M, int N, int K) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * N) return;
    const int m = (int)(idx / N), n = (int)(idx - (int64_t)(idx / N) * N);
    const float* xr = x + (int64_t)m * ldx;
    const float* wr = w + (int64_t)n * K;
    float s = bias ? bias[n] : 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(xr[k], wr[k], s);
    if (r) s += r[(int64_t)m * ldr + n];
    y[(int64_t)m * ldy + n] = s;
}

}  // namespace

namespace {

hipError_t launch_linear_bf16(LinArgs a, hipStream_t stream) {
    // 128x128 tiles when there are enough of them to fill the CUs, else 64x64
    const int64_t big = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128);
    if (big >= 256) {
        a.mtiles = (a.M + 127) / 128;
        a.ntiles = (a.N + 127) / 128;
        if (!grid_fits((int64_t)a.mtiles * a.ntiles)) return hipErrorInvalidConfiguration;
        linear_bf16_kernel<128, 128><<<(unsigned)(a.mtiles * a.ntiles), 256, 0, stream>>>(a);
    } else {
        a.mtiles = (a.M + 63) / 64;
        a.ntiles = (a.N + 63) / 64;
        if (!grid_fits((int64_t)a.mtiles * a.ntiles)) return hipErrorInvalidConfiguration;
        linear_bf16_kernel<64, 64><<<(unsigned)(a.mtiles * a.ntiles), 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(bool bf16, int M, int N, int K, const void* x, int64_t ldx, const void* w,
                         const float* bias, const void* r, int64_t ldr, void* y, int64_t ldy,
                         hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (!bf16) {
        const int64_t total = (int64_t)M * N;
        if (!grid_fits((total + 255) / 256)) return hipErrorInvalidConfiguration;
        linear_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
            (const float*)x, ldx, (const float*)w, bias, (const float*)r, ldr, (float*)y, ldy, M, N, K);
        return hipGetLastError();
    }
    LinArgs a{};
    a.x = (const uint16_t*)x;
    a.w = (const uint16_t*)w;
    a.bias = bias;
    a.r = (const uint16_t*)r;
    a.y = (uint16_t*)y;
    a.ldx = ldx;
    a.ldy = ldy;
    a.ldr = ldr;
    a.M = M;
    a.N = N;
    a.K = K;
    return launch_linear_bf16(a, stream);
}

hipError_t launch_linear_qkv(bool bf16, int M, int N, int K, const void* x, int64_t ldx, const void* w3,
                             const float* bias3, void* const y[3], const int64_t ldy[3], hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (!bf16) {     // the fp32 path: three launches of the same kernel
        for (int sg = 0; sg < 3; ++sg) {
            const hipError_t e = launch_linear(false, M, N, K, x, ldx, (const float*)w3 + (size_t)sg * N * K,
                                               bias3 ? bias3 + (size_t)sg * N : nullptr, nullptr, 0, y[sg],
                                               ldy[sg], stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // one product [M][3N] whose column segments go to the three outputs: each output element is
    // the same K-ordered MFMA sum as in a separate launch
    LinArgs a{};
    a.x = (const uint16_t*)x;
    a.w = (const uint16_t*)w3;
    a.bias = bias3;
    a.y = (uint16_t*)y[0];
    a.y1 = (uint16_t*)y[1];
    a.y2 = (uint16_t*)y[2];
    a.ldx = ldx;
    a.ldy = ldy[0];
    a.ldy1 = ldy[1];
    a.ldy2 = ldy[2];
    a.M = M;
    a.N = 3 * N;
    a.K = K;
    a.segw = N;
    return launch_linear_bf16(a, stream);
}

}  // namespace dp
