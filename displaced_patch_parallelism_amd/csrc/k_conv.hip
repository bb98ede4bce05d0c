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
// bf16 path: implicit GEMM on MFMA (v_mfma_f32_16x16x32_bf16).
//   M = B*h*W output pixels, N = Cout, K = 9*Cin with k = tap*Cin + c, so a
//   K tile of 64 channels lies inside one tap.  Weights [Cout][3][3][Cin] are
//   the GEMM's B^T, row-contiguous in K.  The A loader resolves each pixel's
//   source row once per tap (fresh band / stale map / zero) and streams its
//   128-byte channel runs straight into LDS with direct-to-LDS loads.  Tile
//   128 pixels x 160 channels, 4 waves of 64x80; a 2-stage LDS ring of 36 KB
//   per stage lets two workgroups share a CU so one's waits overlap the
//   other's MFMAs.  Small M is split along K; the fp32 partials are summed in
//   split order by a second kernel (deterministic).
// f32 path: one thread per output element (correctness path for small maps).

#include "dp_device.h"
#include "dp_internal.h"


namespace dp {
namespace {

constexpr int BM = 128;
constexpr int BN = 160;
constexpr int BK = 64;
constexpr int kStages = 2;   // LDS ring depth: 2 x 36 KB, so two workgroups share a CU
constexpr int kWaveKB = 64;  // K tile of the wave-split kernel: 2 stages of 18 KB per wave
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

// ---------------------------------------------------------------------------
// bf16 implicit GEMM, pipelined through LDS with direct-to-LDS loads.
//
// Tile BM=128 pixels x BN output channels, 4 waves in a 2x2 grid, each wave
// 64 pixels x BN/2 channels as 16x16 blocks of v_mfma_f32_16x16x32_bf16.
// Every K tile (64 input channels of one tap) of A (128 rows) and B (BN rows)
// is 128 bytes per row, fetched by global_load_lds_dwordx4 straight into an
// LDS stage (lane l of a load writes the l-th 16-byte slot of a 1 KB chunk).
// The 16-byte chunk c of row r sits at slot c ^ (r & 7) so the MFMA operand
// reads (16 rows x one chunk) spread over the banks.  STAGES stages form a
// ring: while stage k is multiplied, stages k+1.. are in flight.  A rows
// whose source is outside the image (or past the last pixel) read a static
// zero line instead.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

__device__ __attribute__((aligned(64))) uint4 g_zero_line[8];   // never written: reads as zero

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int BN, int STAGES>
__global__ __launch_bounds__(256) void conv3x3_bf16_lds_dma_kernel(ConvArgs a) {
    constexpr int BM2 = 128;
    constexpr int A_CH = BM2 * 128 / 1024;      // 1 KB chunks per A stage (16)
    constexpr int B_CH = BN * 128 / 1024;       // per B stage (BN/8)
    static_assert(A_CH % 4 == 0 && B_CH % 4 == 0, "chunks split over 4 waves");
    constexpr int A_PW = A_CH / 4;
    constexpr int B_PW = B_CH / 4;
    constexpr int LOADS = A_PW + B_PW;          // DMA loads per wave per stage
    constexpr int STAGE = (A_CH + B_CH) * 1024;
    constexpr int WN = BN / 2;                  // channels per wave
    constexpr int NBK = WN / 16;                // 16-wide blocks per wave
    constexpr int SMEM = STAGES * STAGE > BM2 * BN * 4 ? STAGES * STAGE : BM2 * BN * 4;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int mt = blockIdx.x / a.ntiles;
    const int nt = blockIdx.x - mt * a.ntiles;
    const int m0 = mt * BM2;
    const int n0 = nt * BN;
    const int split = blockIdx.y;
    const int kt0 = (int)((int64_t)a.ktiles * split / a.ksplit);
    const int kt1 = (int)((int64_t)a.ktiles * (split + 1) / a.ksplit);
    const int nkt = kt1 - kt0;
    const int cpt = a.Cin / 64;
    const int64_t wrow = 9 * (int64_t)a.Cin;
    const uint16_t* zero = (const uint16_t*)g_zero_line;

    // ---- loader state: this lane's A rows (pixels) and B rows (channels) ----
    const int sub = lane >> 3;          // row within a 1 KB chunk (8 rows of 128 B)
    const int slot = lane & 7;          // physical 16-byte slot in the row
    int pb[A_PW], py[A_PW], px[A_PW], achunk[A_PW];
#pragma unroll
    for (int j = 0; j < A_PW; ++j) {
        const int row = (wave * A_PW + j) * 8 + sub;
        achunk[j] = slot ^ (row & 7);
        const int m = m0 + row;
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
    const uint16_t* bsrc[B_PW];
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
        const int row = (wave * B_PW + j) * 8 + sub;
        const int co = n0 + row;
        const int ch = slot ^ (row & 7);
        bsrc[j] = co < a.Cout ? a.w + co * wrow + ch * 8 : nullptr;
    }
    const uint16_t* asrc[A_PW];
    int cur_tap = -1;

    f32x4 acc[4][NBK];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < NBK; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};

#define DP_ISSUE_STAGE(KT, BUF)                                                                     \
    do {                                                                                            \
        const int kt_ = (KT);                                                                       \
        const int tap_ = kt_ / cpt;                                                                 \
        const int cc_ = kt_ - tap_ * cpt;                                                           \
        const int coff_ = cc_ * 64;                                                                 \
        const int64_t kofs_ = (int64_t)tap_ * a.Cin + coff_;                                        \
        if (tap_ != cur_tap) {                                                                      \
            cur_tap = tap_;                                                                         \
            const int ky_ = tap_ / 3, kx_ = tap_ - 3 * (tap_ / 3);                                  \
            _Pragma("unroll") for (int j = 0; j < A_PW; ++j) {                                      \
                const int r_ = a.r0 + py[j] + ky_ - 1;                                              \
                const int x_ = px[j] + kx_ - 1;                                                     \
                const bool ok_ = pb[j] >= 0 && r_ >= 0 && r_ < a.H && x_ >= 0 && x_ < a.W;          \
                const bool fr_ = r_ >= a.r0 && r_ < a.r0 + a.h;                                     \
                const int64_t fo_ = (((int64_t)pb[j] * a.h + (r_ - a.r0)) * a.W + x_) * a.Cin;      \
                const int64_t so_ = (((int64_t)pb[j] * a.H + r_) * a.W + x_) * a.Cin;               \
                asrc[j] = ok_ ? (fr_ ? a.xp + fo_ : a.xs + so_) + achunk[j] * 8 : nullptr;          \
            }                                                                                       \
        }                                                                                           \
        char* st_ = smem + (BUF) * STAGE;                                                           \
        _Pragma("unroll") for (int j = 0; j < A_PW; ++j) {                                          \
            const uint16_t* g_ = asrc[j] ? asrc[j] + coff_ : zero;                                  \
            __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + (wave * A_PW + j) * 1024), \
                                             16, 0, 0);                                            \
        }                                                                                           \
        _Pragma("unroll") for (int j = 0; j < B_PW; ++j) {                                          \
            const uint16_t* g_ = bsrc[j] ? bsrc[j] + kofs_ : zero;                                  \
            __builtin_amdgcn_global_load_lds((const void*)g_,                                      \
                                             (lds_void*)(st_ + A_CH * 1024 + (wave * B_PW + j) * 1024), \
                                             16, 0, 0);                                            \
        }                                                                                           \
    } while (0)

    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nkt) DP_ISSUE_STAGE(kt0 + s, s);

    // operand read offsets: row (l & 15) of a 16-row block, chunk (ks*4 + l/16) swizzled by (l & 7)
    const int frow = lane & 15;
    const int aoff = (wm * 64 + frow) * 128;
    const int boff = A_CH * 1024 + (wn * WN + frow) * 128;
    const int p0 = ((0 * 4 + (lane >> 4)) ^ (lane & 7)) * 16;
    const int p1 = ((1 * 4 + (lane >> 4)) ^ (lane & 7)) * 16;

    for (int it = 0; it < nkt; ++it) {
        const int ahead = nkt - 1 - it;     // stages issued after this one, capped
        if (ahead >= STAGES - 2)
            wait_vmcnt<(STAGES - 2) * LOADS>();
        else if (STAGES > 3 && ahead == 1)
            wait_vmcnt<LOADS>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (it + STAGES - 1 < nkt) DP_ISSUE_STAGE(kt0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);
        const char* st = smem + (it % STAGES) * STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int po = ks ? p1 : p0;
            bf16x8 af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(st + aoff + i * 16 * 128 + po);
#pragma unroll
            for (int n = 0; n < NBK; ++n) {
                const bf16x8 bfr = *(const bf16x8*)(st + boff + n * 16 * 128 + po);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][n], 0, 0, 0);
            }
        }
    }
#undef DP_ISSUE_STAGE
    __syncthreads();   // all waves done with the ring; reuse it for the output tile

    // ---- epilogue through LDS: lane holds pixel 4*(l/16)+r, channel l%16 of each block ----
    const int ecol = lane & 15;
    const int erow = 4 * (lane >> 4);
    if (a.ksplit == 1) {
        uint16_t* tile = (uint16_t*)smem;   // [BM2][BN] bf16
#pragma unroll
        for (int n = 0; n < NBK; ++n) {
            const int ch = wn * WN + n * 16 + ecol;
            const float bv = (a.bias && n0 + ch < a.Cout) ? a.bias[n0 + ch] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tile[(wm * 64 + i * 16 + erow + r) * BN + ch] = f32_to_bf16(acc[i][n][r] + bv);
        }
        __syncthreads();
        constexpr int CPR = BN * 2 / 16;    // 16-byte chunks per output row
        for (int q = tid; q < BM2 * CPR; q += 256) {
            const int row = q / CPR, c16 = q - (q / CPR) * CPR;
            const int m = m0 + row, co = n0 + c16 * 8;
            if (m < a.M && co < a.Cout)
                *(uint4*)(a.y + (int64_t)m * a.Cout + co) = *(const uint4*)(tile + row * BN + c16 * 8);
        }
    } else {
        float* tile = (float*)smem;         // [BM2][BN] fp32
#pragma unroll
        for (int n = 0; n < NBK; ++n) {
            const int ch = wn * WN + n * 16 + ecol;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) tile[(wm * 64 + i * 16 + erow + r) * BN + ch] = acc[i][n][r];
        }
        __syncthreads();
        constexpr int CPR = BN * 4 / 16;
        float* part = a.part + (int64_t)split * a.M * a.Cout;
        for (int q = tid; q < BM2 * CPR; q += 256) {
            const int row = q / CPR, c16 = q - (q / CPR) * CPR;
            const int m = m0 + row, co = n0 + c16 * 4;
            if (m < a.M && co < a.Cout)
                *(float4*)(part + (int64_t)m * a.Cout + co) = *(const float4*)(tile + row * BN + c16 * 4);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 implicit GEMM for small M: each wave owns a K range.
//
// A workgroup computes one 64-pixel x 80-channel tile; its 4 waves split the
// workgroup's K range into 4 consecutive parts and each wave accumulates the
// whole 64x80 tile (4x5 blocks of v_mfma_f32_16x16x32_bf16) over its part,
// streaming its own A (64 rows) and B (80 rows) K tiles through a private
// 2-stage LDS ring with direct-to-LDS loads -- no barrier in the main loop.
// At the end the four accumulators are added through LDS in wave order
// (deterministic) and the tile is written with coalesced 16-byte stores, as
// bf16 output (+bias) or, when K is also split across workgroups, as fp32
// partials for the ordered reduce kernel.
// ---------------------------------------------------------------------------
constexpr int KS_BM = 64;
constexpr int KS_BN = 80;
constexpr int KS_WAVE_LDS = 36 * 1024;                    // per wave; 4 waves = 144 KB

// KB = K tile width (64: 2 stages of 18 KB; 32: 4 stages of 9 KB per wave).
// Rows of a stage are KB*2 bytes; 16-byte chunk c of row r sits at slot
// c ^ swz(r) (swz = r & 7 for 128-byte rows, (r >> 2) & 3 for 64-byte rows)
// so the 16 rows x 16 bytes of an operand read spread over the LDS banks.
template <int KB>
__global__ __launch_bounds__(256) void conv3x3_bf16_wave_ksplit_kernel(ConvArgs a) {
    constexpr int RB = KB * 2;                          // bytes per row
    constexpr int SLOTS = RB / 16;                      // 16-byte chunks per row
    constexpr int RPC = 1024 / RB;                      // rows per 1 KB DMA chunk
    constexpr int A_CH = KS_BM * RB / 1024;             // DMA chunks per stage for A
    constexpr int B_CH = KS_BN * RB / 1024;             // ... for B
    constexpr int LOADS = A_CH + B_CH;
    constexpr int STAGE = LOADS * 1024;
    constexpr int STAGES = KS_WAVE_LDS / STAGE;         // 2 (KB=64) or 4 (KB=32)
    constexpr int KSTEPS = KB / 32;
    static_assert(STAGES >= 2, "ring depth");
    __shared__ __attribute__((aligned(1024))) char smem[4 * KS_WAVE_LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mt = blockIdx.x / a.ntiles;
    const int nt = blockIdx.x - mt * a.ntiles;
    const int m0 = mt * KS_BM;
    const int n0 = nt * KS_BN;
    const int split = blockIdx.y;
    const int kw0 = (int)((int64_t)a.ktiles * split / a.ksplit);
    const int kw1 = (int)((int64_t)a.ktiles * (split + 1) / a.ksplit);
    const int kt0 = kw0 + (kw1 - kw0) * wave / 4;
    const int kt1 = kw0 + (kw1 - kw0) * (wave + 1) / 4;
    const int nkt = kt1 - kt0;
    const int cpt = a.Cin / KB;
    const int wrow = 9 * a.Cin;
    const uint16_t* zero = (const uint16_t*)g_zero_line;
    char* ring = smem + wave * KS_WAVE_LDS;

    auto swz = [](int row) { return SLOTS == 8 ? (row & 7) : ((row >> 2) & 3); };
    const int sub = lane / SLOTS;
    const int slot = lane % SLOTS;
    int pb[A_CH], py[A_CH], px[A_CH], achunk[A_CH];
#pragma unroll
    for (int j = 0; j < A_CH; ++j) {
        const int row = j * RPC + sub;
        achunk[j] = (slot ^ swz(row)) * 8;
        const int m = m0 + row;
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
    uint32_t boff[B_CH];
#pragma unroll
    for (int j = 0; j < B_CH; ++j) {
        const int row = j * RPC + sub;
        int co = n0 + row;
        if (co >= a.Cout) co = a.Cout - 1;       // clamped rows feed columns that are never stored
        boff[j] = (uint32_t)(((co - n0) * wrow + (slot ^ swz(row)) * 8) * 2);
    }
    const char* wbase = (const char*)(a.w + (int64_t)n0 * wrow);
    const uint16_t* asrc[A_CH];
    int cur_tap = -1;

#define DPK_ISSUE(KT, BUF)                                                                          \
    do {                                                                                            \
        const int kt_ = (KT);                                                                       \
        const int tap_ = kt_ / cpt;                                                                 \
        const int coff_ = (kt_ - tap_ * cpt) * KB;                                                  \
        if (tap_ != cur_tap) {                                                                      \
            cur_tap = tap_;                                                                         \
            const int ky_ = tap_ / 3, kx_ = tap_ - 3 * (tap_ / 3);                                  \
            _Pragma("unroll") for (int j = 0; j < A_CH; ++j) {                                      \
                const int r_ = a.r0 + py[j] + ky_ - 1;                                              \
                const int x_ = px[j] + kx_ - 1;                                                     \
                const bool ok_ = pb[j] >= 0 && r_ >= 0 && r_ < a.H && x_ >= 0 && x_ < a.W;          \
                const bool fr_ = r_ >= a.r0 && r_ < a.r0 + a.h;                                     \
                const int64_t fo_ = (((int64_t)pb[j] * a.h + (r_ - a.r0)) * a.W + x_) * a.Cin;      \
                const int64_t so_ = (((int64_t)pb[j] * a.H + r_) * a.W + x_) * a.Cin;               \
                asrc[j] = ok_ ? (fr_ ? a.xp + fo_ : a.xs + so_) + achunk[j] : nullptr;              \
            }                                                                                       \
        }                                                                                           \
        char* st_ = ring + (BUF) * STAGE;                                                           \
        _Pragma("unroll") for (int j = 0; j < A_CH; ++j) {                                          \
            const uint16_t* g_ = asrc[j] ? asrc[j] + coff_ : zero;   /* padding rows: zero line */ \
            __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + j * 1024), 16, 0, 0); \
        }                                                                                           \
        const char* wk_ = wbase + ((int64_t)tap_ * a.Cin + coff_) * 2;                              \
        _Pragma("unroll") for (int j = 0; j < B_CH; ++j)                                            \
            __builtin_amdgcn_global_load_lds((const void*)(wk_ + boff[j]),                         \
                                             (lds_void*)(st_ + (A_CH + j) * 1024), 16, 0, 0);      \
    } while (0)

    f32x4 acc[4][5];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    int po[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) po[ks] = ((ks * 4 + (lane >> 4)) ^ swz(frow)) * 16;
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nkt) DPK_ISSUE(kt0 + s, s);
    for (int it = 0; it < nkt; ++it) {
        // this wave's stage `it` has landed; later stages may still be in flight
        const int ahead = nkt - 1 - it;
        if (STAGES >= 4 && ahead >= 2) wait_vmcnt<(STAGES >= 4 ? 2 : 0) * LOADS>();
        else if (STAGES >= 3 && ahead >= 1) wait_vmcnt<(STAGES >= 3 ? 1 : 0) * LOADS>();
        else wait_vmcnt<0>();
        if (it + STAGES - 1 < nkt) DPK_ISSUE(kt0 + it + STAGES - 1, (it + STAGES - 1) % STAGES);
        const char* st = ring + (it % STAGES) * STAGE;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            bf16x8 af[4], bfr[5];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(st + (i * 16 + frow) * RB + po[ks]);
#pragma unroll
            for (int n = 0; n < 5; ++n) bfr[n] = *(const bf16x8*)(st + A_CH * 1024 + (n * 16 + frow) * RB + po[ks]);
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], acc[i][n], 0, 0, 0);
        }
    }
#undef DPK_ISSUE
    __syncthreads();   // every wave is done with its ring: reuse the LDS for the reduction

    // acc[i][n][r] = C[pixel i*16 + 4*(l>>4) + r][channel n*16 + (l&15)]
    float* red = (float*)smem;                   // [4 waves][64][80] fp32 (80 KB)
    const int ecol = lane & 15;
    const int erow = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(wave * KS_BM + i * 16 + erow + r) * KS_BN + n * 16 + ecol] = acc[i][n][r];
    __syncthreads();
    // each thread: 4 consecutive channels of 5 (pixel, 4-channel) groups; sum waves in order
    if (a.ksplit == 1) {
        uint16_t* tile = (uint16_t*)(smem + 4 * KS_BM * KS_BN * 4);   // [64][80] bf16 after the fp32 area
        for (int q = tid; q < KS_BM * KS_BN / 4; q += 256) {
            const int row = q / (KS_BN / 4), c4 = (q - row * (KS_BN / 4)) * 4;
            float4 v = *(const float4*)(red + row * KS_BN + c4);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 u = *(const float4*)(red + (w * KS_BM + row) * KS_BN + c4);
                v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
            }
            const int co = n0 + c4;
            if (a.bias && co < a.Cout) {
                v.x += a.bias[co]; v.y += a.bias[co + 1]; v.z += a.bias[co + 2]; v.w += a.bias[co + 3];
            }
            uint2 o;
            o.x = pack_bf16x2(v.x, v.y);
            o.y = pack_bf16x2(v.z, v.w);
            *(uint2*)(tile + row * KS_BN + c4) = o;
        }
        __syncthreads();
        constexpr int CPR = KS_BN * 2 / 16;       // 10 chunks of 16 bytes per row
        for (int q = tid; q < KS_BM * CPR; q += 256) {
            const int row = q / CPR, c16 = q - (q / CPR) * CPR;
            const int m = m0 + row, co = n0 + c16 * 8;
            if (m < a.M && co < a.Cout)
                *(uint4*)(a.y + (int64_t)m * a.Cout + co) = *(const uint4*)(tile + row * KS_BN + c16 * 8);
        }
    } else {
        float* part = a.part + (int64_t)split * a.M * a.Cout;
        for (int q = tid; q < KS_BM * KS_BN / 4; q += 256) {
            const int row = q / (KS_BN / 4), c4 = (q - row * (KS_BN / 4)) * 4;
            float4 v = *(const float4*)(red + row * KS_BN + c4);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 u = *(const float4*)(red + (w * KS_BM + row) * KS_BN + c4);
                v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
            }
            const int m = m0 + row, co = n0 + c4;
            if (m < a.M && co < a.Cout) *(float4*)(part + (int64_t)m * a.Cout + co) = v;
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
    const int64_t M = (int64_t)g.B * g.h * g.W;
    p.ktiles = 9 * g.C / BK;
    const int64_t big_tiles = ((M + BM - 1) / BM) * ((Cout + BN - 1) / BN);
    int ks = 1;
    if (big_tiles >= 128) {
        // enough 128x160 tiles: waves share A and B through LDS; split K if < 256 tiles
        p.kind = 1;
        p.bm = BM;
        p.bn = BN;
        p.mtiles = (int)((M + BM - 1) / BM);
        p.ntiles = (Cout + BN - 1) / BN;
        const int tiles = p.mtiles * p.ntiles;
        if (tiles < 256) {
            ks = (256 + tiles - 1) / tiles;
            const int maxk = p.ktiles / 4 > 0 ? p.ktiles / 4 : 1;
            if (ks > maxk) ks = maxk;
        }
    } else {
        // small M: 64x80 tiles, K split over the 4 waves of a workgroup (and across
        // workgroups until about 256 workgroups, keeping >= 2 K tiles per wave)
        p.kind = 2;
        p.bm = KS_BM;
        p.bn = KS_BN;
        p.ktiles = 9 * g.C / kWaveKB;
        p.mtiles = (int)((M + KS_BM - 1) / KS_BM);
        p.ntiles = (Cout + KS_BN - 1) / KS_BN;
        const int tiles = p.mtiles * p.ntiles;
        if (tiles < 256) {
            ks = (256 + tiles / 2) / tiles;
            const int maxk = p.ktiles / 8 > 0 ? p.ktiles / 8 : 1;
            if (ks > maxk) ks = maxk;
            if (ks < 1) ks = 1;
        }
    }
    if (ks > 32) ks = 32;
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
    if (plan.kind == 2) {
        conv3x3_bf16_wave_ksplit_kernel<kWaveKB><<<grid, kThreads, 0, stream>>>(a);
    }
    else
        conv3x3_bf16_lds_dma_kernel<BN, kStages><<<grid, kThreads, 0, stream>>>(a);
    if (plan.ksplit > 1) {
        const int64_t total4 = (int64_t)a.M * Cout / 4;
        conv_splitk_reduce_kernel<<<(unsigned)((total4 + 255) / 256), 256, 0, stream>>>(
            (const float*)ws, bias, (uint16_t*)y, total4, Cout, plan.ksplit);
    }
    return hipGetLastError();
}

}  // namespace dp
