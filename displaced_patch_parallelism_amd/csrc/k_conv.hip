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
// bf16 path: implicit GEMM on MFMA (v_mfma_f32_16x16x32_bf16), M = output
// pixels, N = Cout, K = 9*Cin, over rectangular pixel tiles (TR rows x 32
// columns of the band) so the three horizontal taps of a kernel row read the
// same source pixels:
//   * The K loop runs over stages (cc, ky): 32 input channels of kernel row
//     ky.  A stage holds the tile's source pixels for that row -- TR rows x 34
//     columns (one extra column each side), 64 bytes each, resolved per pixel
//     to the fresh band, the stale map or zero padding -- and the three taps
//     (ky, 0..2) of the tile's output channels, 64 bytes per (tap, channel).
//     Each source pixel is fetched once per stage instead of once per tap.
//   * Stages are streamed global -> LDS with direct-to-LDS loads
//     (global_load_lds_dwordx4: lane l of a load fills the l-th 16-byte slot of
//     a 1 KB run) through rings of one to three stages.  Slot layout: chunk c
//     (8 channels) of pixel or tap row p sits at slot 4p + (c ^ ((p >> 1) & 3)),
//     which spreads the 16 rows of an MFMA operand read over the banks except
//     that rows p and p + 8 share them (a 2-way conflict; a conflict-free
//     permutation measured no faster).
//   * Weights are read either as given ([Cout][3][3][Cin]) or packed once into
//     [3][Cin/32][3][Cout][32], where a stage's taps are one contiguous block
//     and each 1 KB load reads whole cache lines.
//   * Workgroups are dispatched round-robin over the 8 XCDs; tiles are renumbered
//     so each XCD walks a contiguous run of pixel tiles, keeping the inputs those
//     tiles share in one L2.
//   Large maps: 128x160 tiles (4 rows x 32 columns), one LDS ring shared by
//   4 waves (2x2 of 64 pixels x 80 channels), two workgroups per CU; or, when
//   they fill the GPU in no more rounds, 256x160 tiles (8 rows) with 8 waves,
//   one workgroup per CU and a 3-stage ring.  Small maps: 64x80 tiles (2 rows
//   x 32 columns) whose 8 waves each take an eighth of K through a private
//   buffer and are summed through LDS in wave order; K is also split across
//   workgroups until about 256 of them run, the fp32 partials summed in split
//   order by a second kernel.  Every sum has a fixed order, so results are
//   deterministic.
//   An optional residual (the skip connection of a ResNet block's second conv) is added
//   to acc + bias in fp32 before the single rounding to bf16.
// f32 path: one thread per output element (correctness path for small maps).

#include "dp_device.h"
#include "dp_gn_device.h"
#include "dp_internal.h"


namespace dp {
namespace {

constexpr int kThreads = 256;
constexpr int kTileTC = 32;    // tile columns (both bf16 kernels)

struct ConvArgs {
    const uint16_t* xp;
    const uint16_t* xs;
    const uint16_t* w;
    const float* bias;
    const uint16_t* res;   // residual [B][h][W][Cout] added before rounding, or null
    uint16_t* y;
    float* part;
    int B, H, W, Cin, Cout, h, r0;
    int M;
    int ntx, nty;        // pixel tiles across the band's columns / rows (per batch)
    int mtiles, ntiles;  // pixel tiles (B * nty * ntx), channel tiles
    int kstages;         // K stages (cc, ky): 32 input channels of one kernel row; 3 * Cin / 32
    int ksplit;          // K partitions across workgroups
    int wpacked;         // weights in the packed layout [ky][Cin/32][kx][Cout][32] (else [Cout][3][3][Cin])
    // GroupNorm (+SiLU) applied to the A operand's fresh pixels (the fused kernel only): xp is
    // then the raw GroupNorm input band and xs the conv's stale map, whose band i receives the
    // normalised band (the state the next step reads)
    const float2* gn_part;   // [gn_nblk][B][G] (sum, sum of squares) partials of the band
    const float* gn_stale;   // [P][B][G][2] previous step's moments (null in LOCAL mode)
    const float* gn_gamma;   // [Cin] or null (1)
    const float* gn_beta;    // [Cin] or null (0)
    float* gn_fresh_out;     // [B][G][2] or null
    uint16_t* ystate;        // = xs, writable
    int gn_nblk, gn_G, gn_lanes, gn_mode, gn_silu, gn_P, gn_i;
    float gn_inv_count, gn_eps;
};

// LDS the fused kernel adds after its ring: [lanes][G] lane sums + [G] (mean, rstd), padded to 16
// bytes, then per-channel scale and shift; the host admits the fused kernel only when that fits.
constexpr int kGnFuseLds = 16 * 1024;
__host__ __device__ constexpr int gn_fuse_table_offset(int lanes, int G) { return ((lanes * G + G) * 8 + 15) & ~15; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __attribute__((aligned(64))) uint4 g_zero_line[4];   // never written: reads as zero

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier of the K loops.  Each wave has already waited (explicit vmcnt) for its own
// direct-to-LDS loads of the stage about to be read; the barrier then waits only for the wave's
// own LDS reads and writes.  __syncthreads() would also wait for the loads still in flight into
// the other ring buffers (its fence counts them), leaving the ring a single stage of lookahead.
// The wait sits in the same asm block as the barrier, whose memory clobber keeps the compiler
// from moving memory accesses across the pair.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS accesses of the fused normalisation, written as asm: the compiler's wait insertion takes any
// LDS access for one that may touch the ring buffers the direct-to-LDS loads are still filling, and
// waits for every load in flight before it.  Each thread only touches the slots its own loads
// filled (waited for explicitly) and the parameter table.  One block per stage reads the thread's
// 8 channels of scale and shift (t, t + 16 bytes; shift at u) and its three A slots (a, a + 8 KB,
// a + 16 KB) and waits for them; the writes carry no memory clobber, so the compiler may move the
// MFMAs' own LDS reads around them (they touch another ring buffer).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }
__device__ __forceinline__ void lds_read_xform(uint32_t t, uint32_t u, uint32_t a, u32x4& s0, u32x4& s1, u32x4& f0,
                                               u32x4& f1, u32x4& r0, u32x4& r1, u32x4& r2) {
    asm volatile(
        "ds_read_b128 %0, %7\n\tds_read_b128 %1, %7 offset:16\n\t"
        "ds_read_b128 %2, %8\n\tds_read_b128 %3, %8 offset:16\n\t"
        "ds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:8192\n\tds_read_b128 %6, %9 offset:16384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(s0), "=&v"(s1), "=&v"(f0), "=&v"(f1), "=&v"(r0), "=&v"(r1), "=&v"(r2)
        : "v"(t), "v"(u), "v"(a));
}
template <int Q>
__device__ __forceinline__ void lds_write_slot(uint32_t a, u32x4 v) {
    static_assert(Q >= 0 && Q < 3, "three A slots per thread");
    if constexpr (Q == 0) asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v));
    else if constexpr (Q == 1) asm volatile("ds_write_b128 %0, %1 offset:8192" ::"v"(a), "v"(v));
    else asm volatile("ds_write_b128 %0, %1 offset:16384" ::"v"(a), "v"(v));
}

__device__ __forceinline__ int slot_swz(int p) { return (p >> 1) & 3; }

// Geometry of one stage for a TR x 32 pixel tile and BN output channels.
template <int TR, int BN>
struct Stage {
    static constexpr int HWC = kTileTC + 2;                 // halo columns
    static constexpr int A_SLOTS = TR * HWC * 4;            // 16-byte slots of source pixels
    static constexpr int A_LOADS = (A_SLOTS + 63) / 64;     // 1 KB direct-to-LDS loads
    static constexpr int A_TAIL = A_SLOTS - (A_LOADS - 1) * 64;   // active lanes of the last one
    static constexpr int B_SLOTS = 3 * BN * 4;              // three taps x BN channel rows
    static constexpr int B_LOADS = B_SLOTS / 64;
    static constexpr int B_OFF = A_SLOTS * 16;
    static constexpr int BYTES = (A_SLOTS + B_SLOTS) * 16;
    static_assert(B_SLOTS % 64 == 0 && BN % 80 == 0, "channel tile");
};

// Workgroup b runs on XCD b % 8: give XCD x the contiguous run x*q + min(x, r) .. of the
// logical tile order (q = total / 8, r = total % 8).  A bijection of [0, total).
__device__ __forceinline__ int xcd_order(int b, int total) {
    const int x = b & 7, i = b >> 3;
    const int q = total >> 3, r = total & 7;
    return x * q + (x < r ? x : r) + i;
}

// Source of A slot s of a stage of tile (bb, ty0, tx0), for kernel rows ky = 0, 1, 2:
// pointer to channel chunk c of the pixel, or null where the pixel is zero padding.  Offsets
// inside one batch image are 32-bit (the host rejects images of 2^31 or more elements).
template <int TR>
__device__ __forceinline__ void resolve_a_slot(const ConvArgs& a, int bb, int ty0, int tx0, int s,
                                               const uint16_t*& p0, const uint16_t*& p1,
                                               const uint16_t*& p2) {
    constexpr int HWC = kTileTC + 2;
    const int p = s >> 2;
    const int t = p / HWC, u = p - t * HWC;
    const int c = (s & 3) ^ slot_swz(p);
    const int x = tx0 + u - 1;
    const bool xok = s < TR * HWC * 4 && x >= 0 && x < a.W;
    const uint16_t* fb = a.xp + (int64_t)bb * a.h * a.W * a.Cin;     // this batch image's band
    const uint16_t* sb = a.xs + (int64_t)bb * a.H * a.W * a.Cin;     // and stale map
    const uint16_t* q[3];
#pragma unroll
    for (int ky = 0; ky < 3; ++ky) {
        const int r = a.r0 + ty0 + t + ky - 1;    // image row feeding tile row t through kernel row ky
        const bool ok = xok && r >= 0 && r < a.H;
        const bool fresh = r >= a.r0 && r < a.r0 + a.h;
        const uint32_t pix = (uint32_t)((fresh ? r - a.r0 : r) * a.W + x);
        const uint32_t off = pix * (uint32_t)a.Cin + (uint32_t)(c * 8);
        q[ky] = ok ? (fresh ? fb : sb) + off : nullptr;
    }
    p0 = q[0];
    p1 = q[1];
    p2 = q[2];
}

// Byte offset of this lane's slot in B load j (tap rows 16j .. 16j+15, 4 chunks each) from the
// stage's weights.  BN is a multiple of 16, so the load's tap kx and the rows' swizzle
// ((16j + lane/4) >> 1) & 3 = (lane >> 3) & 3 do not depend on the row.
template <int BN>
__device__ __forceinline__ uint32_t b_slot_offset(const ConvArgs& a, int n0, int j, int lane) {
    static_assert(BN % 16 == 0, "B loads cover whole 16-row groups of one tap");
    const int kx = (16 * j) / BN;
    const int n = 16 * j - kx * BN + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 3) & 3);
    int co = n0 + n;
    if (co >= a.Cout) co = a.Cout - 1;      // clamped rows feed columns that are never stored
    if (a.wpacked) return (uint32_t)(((kx * a.Cout + co) * 32 + c * 8) * 2);
    return (uint32_t)(((co * 9 + kx) * a.Cin + c * 8) * 2);
}

// First byte of stage (cc, ky)'s weights; b_slot_offset is relative to it.  In the packed
// layout a stage is one contiguous block of 3 x Cout rows of 64 bytes, so the 16 tap rows one
// direct-to-LDS load fills are 1 KB of consecutive memory (whole cache lines).
__device__ __forceinline__ const char* stage_weights(const ConvArgs& a, int cc, int ky) {
    if (a.wpacked) return (const char*)a.w + ((int64_t)ky * (a.Cin / 32) + cc) * 3 * a.Cout * 64;
    return (const char*)a.w + ((int64_t)3 * ky * a.Cin + cc * 32) * 2;
}

// The 60 MFMAs of one stage for a wave's 64 pixels (tile rows tr0, tr0+1, 32 columns) x 80
// channels.  aoff[r][kx]: byte offset of this lane's operand row for tile row tr0+r, columns
// 0..15, tap kx; columns 16..31 are 1 KB further.  boff: this lane's operand row of tap 0,
// channel block 0 of the wave; tap kx, block n are (kx*BN + 16n) * 64 bytes further.
template <int BN>
__device__ __forceinline__ void stage_mfma(const char* st, const int (&aoff)[2][3], int boff,
                                           f32x4 (&acc)[4][5]) {
#pragma unroll
    for (int kx = 0; kx < 3; ++kx) {
        bf16x8 af[4], bfr[5];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(st + aoff[i >> 1][kx] + (i & 1) * 1024);
#pragma unroll
        for (int n = 0; n < 5; ++n) bfr[n] = *(const bf16x8*)(st + boff + (kx * BN + n * 16) * 64);
#pragma unroll
        for (int n = 0; n < 5; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], acc[i][n], 0, 0, 0);
    }
}

// Operand read offsets of this lane for a wave whose pixels are tile rows tr0, tr0+1.
template <int TR, int BN>
__device__ __forceinline__ void operand_offsets(int lane, int tr0, int wn, int (&aoff)[2][3], int& boff) {
    constexpr int HWC = kTileTC + 2;
    const int row = lane & 15, ch = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) {
            const int p = (tr0 + r) * HWC + kx + row;
            aoff[r][kx] = (4 * p + (ch ^ slot_swz(p))) * 16;
        }
    boff = Stage<TR, BN>::B_OFF + (4 * (wn * 80 + row) + (ch ^ slot_swz(row))) * 16;
}

// Decode a tile index: batch, first band row, first column.
template <int TR>
__device__ __forceinline__ void tile_origin(const ConvArgs& a, int mt, int& bb, int& ty0, int& tx0) {
    const int txt = mt % a.ntx;
    const int rest = mt / a.ntx;
    const int tyt = rest % a.nty;
    bb = rest / a.nty;
    ty0 = tyt * TR;
    tx0 = txt * kTileTC;
}

// ---------------------------------------------------------------------------
// Large maps: tile TR rows x 32 columns x 160 channels; NW = TR waves (TR/2 pixel-row pairs x 2
// channel halves of 64 pixels x 80 channels each) share one STAGES-deep ring; a barrier per
// stage publishes it.  The stage's loads are dealt round-robin to the waves.
//   TR = 4: 4 waves, 2 x 38.5 KB, two workgroups per CU (one's waits overlap the other's MFMAs).
//   TR = 8: 8 waves, 3 x 47 KB, one workgroup per CU: the 160 channels' weights of a stage serve
//           256 pixels instead of 128, and two stages load while one is multiplied; the
//           GroupNorm-folding conv's tile (its lanes and parameter table take the LDS left over).
// ---------------------------------------------------------------------------
// Fused GroupNorm: which kernel rows ky = 0..2 read slot s of a stage from the fresh band (bit ky
// of the mask), and, for a fresh pixel of the tile's own columns in its own rows (kernel row 1)
// of channel tile 0, where its normalised value goes in the conv's stale map (else null).
template <int TR>
__device__ __forceinline__ void fuse_slot(const ConvArgs& a, int bb, int ty0, int tx0, int s, bool own_tile,
                                          uint32_t& fmask, uint16_t*& ysp) {
    constexpr int HWC = kTileTC + 2;
    const int p = s >> 2;
    const int t = p / HWC, u = p - t * HWC;
    const int c = (s & 3) ^ slot_swz(p);
    const int x = tx0 + u - 1;
    const bool xok = s < TR * HWC * 4 && x >= 0 && x < a.W;
    fmask = 0;
#pragma unroll
    for (int ky = 0; ky < 3; ++ky) {
        const int r = a.r0 + ty0 + t + ky - 1;
        if (xok && r >= a.r0 && r < a.r0 + a.h) fmask |= 1u << ky;
    }
    ysp = nullptr;
    if (own_tile && (fmask & 2u) && u >= 1 && u <= kTileTC)
        ysp = a.ystate + (((int64_t)bb * a.H + a.r0 + ty0 + t) * a.W + x) * a.Cin + c * 8;
}

template <int TR, int STAGES, bool FUSE>
__device__ __forceinline__ void conv_tile_body(const ConvArgs& a, char* smem) {
    constexpr int BN = 160;
    constexpr int NW = TR;                        // waves: TR / 2 row pairs x 2 channel halves
    using S = Stage<TR, BN>;
    constexpr int AQ = (S::A_LOADS + NW - 1) / NW;   // A loads per wave (at most)
    constexpr int BQ = (S::B_LOADS + NW - 1) / NW;
    constexpr int PX = TR * kTileTC;              // output pixels per tile

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % (TR / 2), wn = wave / (TR / 2);
    const int lt = xcd_order(blockIdx.x, gridDim.x);
    // channel tile fastest: the workgroups of one pixel tile run on one XCD, which then fetches
    // the tile's source pixels once for all of them (its L2 holds every channel tile's weights)
    const int nt = lt % a.ntiles;
    const int mt = lt / a.ntiles;
    int bb, ty0, tx0;
    tile_origin<TR>(a, mt, bb, ty0, tx0);
    const int n0 = nt * BN;
    const uint16_t* zero = (const uint16_t*)g_zero_line;

    const uint16_t* ap0[AQ];
    const uint16_t* ap1[AQ];
    const uint16_t* ap2[AQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int j = wave + NW * q;
        resolve_a_slot<TR>(a, bb, ty0, tx0, j * 64 + lane, ap0[q], ap1[q], ap2[q]);
    }
    uint32_t bo[BQ];
#pragma unroll
    for (int q = 0; q < BQ; ++q) bo[q] = b_slot_offset<BN>(a, n0, wave + NW * q, lane);
    // this wave's loads per stage (the deal is uneven when NW does not divide the load counts)
    const int nloads = (S::A_LOADS - wave + NW - 1) / NW + (S::B_LOADS - wave + NW - 1) / NW;
    // fused GroupNorm: each thread normalises the fresh pixels its own A loads brought in (all of
    // a thread's slots hold the same 8-channel chunk cthr of their pixel)
    uint32_t fmask[AQ];
    uint16_t* ysp[AQ];
    const int cthr = (lane & 3) ^ ((lane >> 3) & 3);
    if constexpr (FUSE) {
        static_assert(AQ == 3 && NW == 8, "three A loads 8 KB apart per thread: one normalised per tap");
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const int j = wave + NW * q;
            fmask[q] = 0;
            ysp[q] = nullptr;
            if (j < S::A_LOADS) fuse_slot<TR>(a, bb, ty0, tx0, j * 64 + lane, nt == 0, fmask[q], ysp[q]);
        }
    }

    // Issue the loads of stage (cc, KY) into ring buffer BUF; KY is a literal so each kernel row
    // reads its own source array (a runtime select between them becomes a scratch-indexed load).
#define DPH_ISSUE_KY(CC, KY, SRC, BUF)                                                              \
    do {                                                                                            \
        char* st_ = smem + (BUF) * S::BYTES;                                                        \
        _Pragma("unroll") for (int q = 0; q < AQ; ++q) {                                            \
            const int j_ = wave + NW * q;                                                           \
            if (j_ < S::A_LOADS) {                                                                  \
                const uint16_t* g_ = SRC[q] ? SRC[q] + (CC) * 32 : zero;                            \
                if (j_ < S::A_LOADS - 1 || lane < S::A_TAIL)                                        \
                    __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + j_ * 1024), \
                                                     16, 0, 0);                                    \
            }                                                                                       \
        }                                                                                           \
        const char* wk_ = stage_weights(a, (CC), (KY));                                           \
        _Pragma("unroll") for (int q = 0; q < BQ; ++q) {                                            \
            const int j_ = wave + NW * q;                                                           \
            if (j_ < S::B_LOADS)                                                                    \
                __builtin_amdgcn_global_load_lds((const void*)(wk_ + bo[q]),                       \
                                                 (lds_void*)(st_ + S::B_OFF + j_ * 1024), 16, 0, 0); \
        }                                                                                           \
    } while (0)
#define DPH_ISSUE(K, BUF)                                                                           \
    do {                                                                                            \
        const int cc_ = (K) / 3;                                                                    \
        switch ((K) - 3 * cc_) {                                                                    \
            case 0: DPH_ISSUE_KY(cc_, 0, ap0, BUF); break;                                          \
            case 1: DPH_ISSUE_KY(cc_, 1, ap1, BUF); break;                                          \
            default: DPH_ISSUE_KY(cc_, 2, ap2, BUF); break;                                         \
        }                                                                                           \
    } while (0)

    f32x4 acc[4][5];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    int aoff[2][3], boff;
    operand_offsets<TR, BN>(lane, 2 * wm, wn, aoff, boff);

    const int nk = a.kstages;
#pragma unroll
    for (int k = 0; k < STAGES - 1; ++k)
        if (k < nk) DPH_ISSUE(k, k);

    if constexpr (FUSE) {
        static_assert(STAGES == 3, "the fused kernel normalises stage it+1 while it multiplies stage it");
        // ---- the band's GroupNorm parameters, while the first stages load: the same partial
        // sums, in the same order, as the normalising kernel's (so the normalised values are
        // bitwise those of the two-kernel path) ----
        const int G = a.gn_G, L = a.gn_lanes;
        float2* gred = (float2*)(smem + STAGES * S::BYTES);    // [L][G]
        float2* gmr = gred + L * G;                             // [G] (mean, rstd)
        float* tsc = (float*)(smem + STAGES * S::BYTES + gn_fuse_table_offset(L, G));   // [Cin] scale
        float* tsf = tsc + a.Cin;                               // [Cin] shift
        if (tid < L * G) {
            const int g = tid % G, j0 = tid / G;
            float sa = 0.f, sq = 0.f;
            for (int jb = j0; jb < a.gn_nblk; jb += 8 * L) {
                float2 pv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = jb + u * L;
                    pv[u] = j < a.gn_nblk ? a.gn_part[((int64_t)j * a.B + bb) * G + g] : make_float2(0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    sa += pv[u].x;
                    sq += pv[u].y;
                }
            }
            gred[j0 * G + g] = make_float2(sa, sq);
        }
        __syncthreads();
        if (tid < G) {
            const int g = tid;
            float sa = 0.f, sq = 0.f;
            for (int k = 0; k < L; ++k) {
                sa += gred[k * G + g].x;
                sq += gred[k * G + g].y;
            }
            float st_e = 0.f, st_q = 0.f;
            if (a.gn_mode != 1) {
                for (int j = 0; j < a.gn_P; ++j) {
                    if (a.gn_mode == 0 && j == a.gn_i) continue;
                    st_e += a.gn_stale[(((int64_t)j * a.B + bb) * G + g) * 2 + 0];
                    st_q += a.gn_stale[(((int64_t)j * a.B + bb) * G + g) * 2 + 1];
                }
            }
            const float m = sa * a.gn_inv_count, qm = sq * a.gn_inv_count;
            if (a.gn_fresh_out && nt == 0 && ty0 == 0 && tx0 == 0) {   // one workgroup per batch image
                a.gn_fresh_out[(bb * G + g) * 2 + 0] = m;
                a.gn_fresh_out[(bb * G + g) * 2 + 1] = qm;
            }
            gmr[g] = gn_group_norm_params(m, qm, st_e, st_q, a.gn_mode, a.gn_P, a.gn_eps);
        }
        __syncthreads();
        const int cg = a.Cin / G;
        for (int c = tid; c < a.Cin; c += 64 * NW)
            gn_scale_shift(gmr[c / cg], a.gn_gamma ? a.gn_gamma[c] : 1.f, a.gn_beta ? a.gn_beta[c] : 0.f, tsc[c],
                           tsf[c]);
        __syncthreads();
    }
    // Stage K's table entries and this thread's three A slots (ring buffer BUF), in registers
#define DPH_XFORM_LOAD(K, BUF)                                                                      \
    do {                                                                                            \
        const float* gt_ = (const float*)(smem + STAGES * S::BYTES + gn_fuse_table_offset(a.gn_lanes, a.gn_G)); \
        const int ch_ = ((K) / 3) * 32 + cthr * 8;                                                  \
        xsa_ = lds_addr(smem + (BUF) * S::BYTES + wave * 1024 + lane * 16);                          \
        u32x4 s0_, s1_, f0_, f1_;                                                                   \
        lds_read_xform(lds_addr(gt_ + ch_), lds_addr(gt_ + a.Cin + ch_), xsa_, s0_, s1_, f0_, f1_, xr_[0], xr_[1], \
                       xr_[2]);                                                                     \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                             \
            xsc_[e] = __uint_as_float(s0_[e]);                                                      \
            xsc_[e + 4] = __uint_as_float(s1_[e]);                                                  \
            xsf_[e] = __uint_as_float(f0_[e]);                                                      \
            xsf_[e + 4] = __uint_as_float(f1_[e]);                                                  \
        }                                                                                           \
    } while (0)
    // the fresh pixels of this thread's slot of load Q in stage K, normalised in place; those of the
    // tile's own rows and columns (kernel row 1) also go to the stale map
#define DPH_XFORM_Q(K, Q)                                                                           \
    do {                                                                                            \
        const int ky_ = (K) % 3;                                                                    \
        if ((fmask[Q] >> ky_) & 1u) {                                                               \
            float f_[8];                                                                            \
            unpack8(make_uint4(xr_[Q][0], xr_[Q][1], xr_[Q][2], xr_[Q][3]), f_);                    \
            _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                         \
                float z_ = fmaf(f_[e], xsc_[e], xsf_[e]);                                           \
                if (a.gn_silu) z_ = silu(z_);                                                       \
                f_[e] = z_;                                                                         \
            }                                                                                       \
            const uint4 v_ = pack8(f_);                                                             \
            lds_write_slot<Q>(xsa_, u32x4{v_.x, v_.y, v_.z, v_.w});                                 \
            if (ky_ == 1 && ysp[Q]) *(uint4*)(ysp[Q] + ((K) / 3) * 32) = v_;                        \
        }                                                                                           \
    } while (0)
    float xsc_[8], xsf_[8];      // scale and shift of this thread's 8 channels of one stage
    u32x4 xr_[3];                // this thread's three A slots of that stage
    uint32_t xsa_ = 0;           // LDS address of its first slot
    if constexpr (FUSE) {
        if (nk > 0) {
            // this wave's loads of stage 0 have landed (stage 1's may still be in flight)
            if (nk > 1) {
                if (nloads >= 7) wait_vmcnt<7>();
                else if (nloads == 6) wait_vmcnt<6>();
                else if (nloads == 5) wait_vmcnt<5>();
                else wait_vmcnt<0>();
            } else {
                wait_vmcnt<0>();
            }
            DPH_XFORM_LOAD(0, 0);
            DPH_XFORM_Q(0, 0);
            DPH_XFORM_Q(0, 1);
            DPH_XFORM_Q(0, 2);
        }
        for (int it = 0; it < nk; ++it) {
            ring_barrier();      // stage it normalised by every thread; everyone is done with stage it-1
            if (it + 2 < nk) DPH_ISSUE(it + 2, (it + 2) % 3);
            const bool nxt = it + 1 < nk;
            if (nxt) {           // this wave's loads of stage it+1 have landed (stage it+2's may not)
                if (it + 2 < nk) {
                    if (nloads >= 7) wait_vmcnt<7>();
                    else if (nloads == 6) wait_vmcnt<6>();
                    else if (nloads == 5) wait_vmcnt<5>();
                    else wait_vmcnt<0>();
                } else {
                    wait_vmcnt<0>();
                }
                DPH_XFORM_LOAD(it + 1, (it + 1) % 3);
            }
            // stage it's 60 MFMAs, tap by tap, with stage it+1's normalisation between the taps
            const char* st = smem + (it % 3) * S::BYTES;
#pragma unroll
            for (int kx = 0; kx < 3; ++kx) {
                bf16x8 af[4], bfr[5];
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(st + aoff[i >> 1][kx] + (i & 1) * 1024);
#pragma unroll
                for (int n = 0; n < 5; ++n) bfr[n] = *(const bf16x8*)(st + boff + (kx * BN + n * 16) * 64);
                if (nxt) {
                    if (kx == 0) DPH_XFORM_Q(it + 1, 0);
                    else if (kx == 1) DPH_XFORM_Q(it + 1, 1);
                    else DPH_XFORM_Q(it + 1, 2);
                }
#pragma unroll
                for (int n = 0; n < 5; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], acc[i][n], 0, 0, 0);
            }
        }
    }
    for (int it = 0; it < (FUSE ? 0 : nk); ++it) {
        // this wave's loads of stage it have landed (those of the stages after it, issued later,
        // may still be in flight; loads complete in order) ...
        if (STAGES == 2 || it + 1 >= nk) {
            wait_vmcnt<0>();
        } else {
            static_assert(STAGES == 2 || STAGES == 3, "ring depth");
            // one later stage in flight: allow this wave's per-stage load count
            if (nloads >= 7) wait_vmcnt<7>();
            else if (nloads == 6) wait_vmcnt<6>();
            else if (nloads == 5) wait_vmcnt<5>();
            else wait_vmcnt<0>();
        }
        ring_barrier();      // ... and everyone's; everyone is also done with stage it-1
        if (it + STAGES - 1 < nk) DPH_ISSUE(it + STAGES - 1, (it + STAGES - 1) % STAGES);
        stage_mfma<BN>(smem + (it % STAGES) * S::BYTES, aoff, boff, acc);
    }
#undef DPH_ISSUE
#undef DPH_ISSUE_KY
#undef DPH_XFORM_LOAD
#undef DPH_XFORM_Q
    __syncthreads();   // ring no longer read: reuse it for the output tile

    // acc[i][n][r] = D[pixel 16i + 4(l>>4) + r of the wave][channel 16n + (l&15) of the wave]
    const int ecol = lane & 15;
    const int erow = 4 * (lane >> 4);
    if (a.res) {
        // acc + bias staged in fp32, one channel half (the waves of wn = pass) at a time (the
        // whole fp32 tile would not fit the ring); the residual is added before rounding
        float* ft = (float*)smem;            // [PX pixels][80 + 4] fp32 (padded pitch)
        constexpr int FP = 84;
        static_assert(PX * FP * 4 <= STAGES * S::BYTES, "fp32 half tile fits the ring");
        for (int pass = 0; pass < 2; ++pass) {
            if (pass) __syncthreads();       // the previous half has been read
            if (wn == pass) {
#pragma unroll
                for (int n = 0; n < 5; ++n) {
                    const int ch = n * 16 + ecol;
                    const float bv = (a.bias && n0 + pass * 80 + ch < a.Cout) ? a.bias[n0 + pass * 80 + ch] : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) ft[(wm * 64 + i * 16 + erow + r) * FP + ch] = acc[i][n][r] + bv;
                }
            }
            __syncthreads();
            for (int q = tid; q < PX * 10; q += 64 * NW) {
                const int px = q / 10, c8 = q - px * 10;
                const int y = ty0 + (px >> 5), x = tx0 + (px & 31), co = n0 + pass * 80 + c8 * 8;
                if (y < a.h && x < a.W && co < a.Cout) {
                    const int64_t o = (((int64_t)bb * a.h + y) * a.W + x) * a.Cout + co;
                    const float4 lo = *(const float4*)(ft + px * FP + c8 * 8);
                    const float4 hi = *(const float4*)(ft + px * FP + c8 * 8 + 4);
                    float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    float rv[8];
                    unpack8(*(const uint4*)(a.res + o), rv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] += rv[e];
                    *(uint4*)(a.y + o) = pack8(f);
                }
            }
        }
        return;
    }
    uint16_t* tile = (uint16_t*)smem;    // [PX pixels][BN] bf16, pixel = tile row * 32 + column
#pragma unroll
    for (int n = 0; n < 5; ++n) {
        const int ch = wn * 80 + n * 16 + ecol;
        const float bv = (a.bias && n0 + ch < a.Cout) ? a.bias[n0 + ch] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tile[(wm * 64 + i * 16 + erow + r) * BN + ch] = f32_to_bf16(acc[i][n][r] + bv);
    }
    __syncthreads();
    constexpr int CPR = BN * 2 / 16;    // 16-byte chunks per output pixel
    for (int q = tid; q < PX * CPR; q += 64 * NW) {
        const int px = q / CPR, c16 = q - px * CPR;
        const int y = ty0 + (px >> 5), x = tx0 + (px & 31), co = n0 + c16 * 8;
        if (y < a.h && x < a.W && co < a.Cout)
            *(uint4*)(a.y + (((int64_t)bb * a.h + y) * a.W + x) * a.Cout + co) =
                *(const uint4*)(tile + px * BN + c16 * 8);
    }
}

template <int TR, int STAGES>
constexpr int tile_smem() {
    using S = Stage<TR, 160>;
    return STAGES * S::BYTES > TR * kTileTC * 160 * 2 ? STAGES * S::BYTES : TR * kTileTC * 160 * 2;
}

__global__ __launch_bounds__(256, 2) void conv3x3_bf16_halo_tile_kernel(ConvArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[tile_smem<4, 2>()];
    conv_tile_body<4, 2, false>(a, smem);
}

// The 256x160-tile conv whose A operand's fresh pixels are the raw GroupNorm input, normalised
// (+ SiLU) on the fly: GroupNorm-apply fused into the conv (the statistics pass runs before it).
// Halo rows come from the conv's stale map, already normalised by the previous step; zero padding
// stays zero.  Channel tile 0 also writes the normalised band into band i of that map.
__global__ __launch_bounds__(512, 1) void conv3x3_bf16_gn_tile8_kernel(ConvArgs a) {
    static_assert(tile_smem<8, 3>() + kGnFuseLds <= 160 * 1024, "LDS of one workgroup");
    __shared__ __attribute__((aligned(1024))) char smem[tile_smem<8, 3>() + kGnFuseLds];
    conv_tile_body<8, 3, true>(a, smem);
}

// ---------------------------------------------------------------------------
// Small maps: tile 2 rows x 32 columns x 80 channels with K split over 8 waves (two per SIMD),
// and across workgroups until about 256 of them run (fp32 partials, summed in split order by
// conv_splitk_reduce_kernel).  Each wave streams its stages through a single private buffer, refilled
// tap by tap: once tap kx's fragments are in registers, the next stage's weight rows of tap kx go
// into the freed rows (and after the last tap, its source pixels), then tap kx's 20 MFMAs run, so
// two thirds of the refill are in flight a tap or two earlier than a whole-stage refill would be.
// A wave stalls while the CU's vector memory path takes its loads; the other wave on its SIMD
// multiplies meanwhile.  The 8 accumulators are summed through LDS in wave order (the whole
// 160 KB holds 8 x 64 x 80 fp32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void conv3x3_bf16_halo_wave8_kernel(ConvArgs a) {
    constexpr int TR = 2, BN = 80, NW = 8;
    using S = Stage<TR, BN>;
    constexpr int RED = 64 * BN * 4;                 // one wave's fp32 partial tile
    static_assert(S::BYTES <= RED, "a wave's stage buffer lies inside its reduction slot");
    __shared__ __attribute__((aligned(1024))) char smem[NW * RED];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, so the wave's K range, stage indices and LDS buffer stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // logical order (channel tile, K split, pixel tile), pixel tile fastest
    const int lt = xcd_order(blockIdx.x, gridDim.x);
    const int mt = lt % a.mtiles;
    const int rest = lt / a.mtiles;
    const int split = rest % a.ksplit;
    const int nt = rest / a.ksplit;
    const int n0 = nt * BN;
    // kstages * ksplit < 2^31 for every conv the host accepts (weights under 2 GiB, <= 32 splits)
    const int k0 = a.kstages * split / a.ksplit;
    const int k1 = a.kstages * (split + 1) / a.ksplit;
    const int kb = k0 + (k1 - k0) * wave / NW;
    const int nk = k0 + (k1 - k0) * (wave + 1) / NW - kb;
    const uint16_t* zero = (const uint16_t*)g_zero_line;
    char* buf = smem + wave * RED;

    // B slot offsets of tap 0; tap kx's are kx * kxs further (the clamped row depends on the row only)
    uint32_t bo[BN / 16];
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) bo[j] = b_slot_offset<BN>(a, n0, j, lane);
    const int64_t kxs = a.wpacked ? (int64_t)a.Cout * 64 : (int64_t)a.Cin * 2;

    // a stage in parts: the B loads of tap KX (tap rows KX*BN .. +BN-1), and the A loads
#define DP8_ISSUE_B(K, KX)                                                                          \
    do {                                                                                            \
        const int cc_ = (K) / 3;                                                                    \
        const char* wk_ = stage_weights(a, cc_, (K) - 3 * cc_) + (KX) * kxs;                        \
        _Pragma("unroll") for (int j = 0; j < BN / 16; ++j)                                         \
            __builtin_amdgcn_global_load_lds((const void*)(wk_ + bo[j]),                           \
                                             (lds_void*)(buf + S::B_OFF + ((KX) * (BN / 16) + j) * 1024), \
                                             16, 0, 0);                                             \
    } while (0)
#define DP8_ISSUE_A_KY(CC, SRC)                                                                     \
    do {                                                                                            \
        _Pragma("unroll") for (int j = 0; j < S::A_LOADS; ++j) {                                    \
            const uint16_t* g_ = SRC[j] ? SRC[j] + (CC) * 32 : zero;                                \
            if (j < S::A_LOADS - 1 || lane < S::A_TAIL)                                             \
                __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(buf + j * 1024), 16, 0, 0); \
        }                                                                                           \
    } while (0)
#define DP8_ISSUE_A(K)                                                                              \
    do {                                                                                            \
        const int cc_ = (K) / 3;                                                                    \
        switch ((K) - 3 * cc_) {                                                                    \
            case 0: DP8_ISSUE_A_KY(cc_, ap0); break;                                                \
            case 1: DP8_ISSUE_A_KY(cc_, ap1); break;                                                \
            default: DP8_ISSUE_A_KY(cc_, ap2); break;                                               \
        }                                                                                           \
    } while (0)

    f32x4 acc[4][5];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    int aoff[2][3], boff;
    operand_offsets<TR, BN>(lane, 0, 0, aoff, boff);

    // the first stage's weight rows go out before the source pixels are resolved (their
    // addresses are a few operations; the pixels' take most of the prologue)
    if (nk > 0) {
        DP8_ISSUE_B(kb, 0);
        DP8_ISSUE_B(kb, 1);
        DP8_ISSUE_B(kb, 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    int bb, ty0, tx0;
    tile_origin<TR>(a, mt, bb, ty0, tx0);
    const uint16_t* ap0[S::A_LOADS];
    const uint16_t* ap1[S::A_LOADS];
    const uint16_t* ap2[S::A_LOADS];
#pragma unroll
    for (int j = 0; j < S::A_LOADS; ++j) resolve_a_slot<TR>(a, bb, ty0, tx0, j * 64 + lane, ap0[j], ap1[j], ap2[j]);
    if (nk > 0) DP8_ISSUE_A(kb);
    for (int it = 0; it < nk; ++it) {
        wait_vmcnt<0>();     // stage it has landed in this wave's buffer
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) {
            bf16x8 af[4], bfr[5];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(buf + aoff[i >> 1][kx] + (i & 1) * 1024);
#pragma unroll
            for (int n = 0; n < 5; ++n) bfr[n] = *(const bf16x8*)(buf + boff + (kx * BN + n * 16) * 64);
            // tap kx's fragments are in registers: its B rows may take the next stage's (and after
            // the last tap, so may the A pixels)
            __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): every read above has returned
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < nk) {
                if (kx == 2) DP8_ISSUE_A(kb + it + 1);
                DP8_ISSUE_B(kb + it + 1, kx);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < 5; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[n], acc[i][n], 0, 0, 0);
        }
    }
#undef DP8_ISSUE_B
#undef DP8_ISSUE_A
#undef DP8_ISSUE_A_KY
    // the bias of the channels this thread stores below, loaded now so that its latency
    // overlaps the partial-tile exchange (in the loop each load would be waited out in turn)
    constexpr int G4 = 64 * BN / 4;                  // 4-channel groups of the tile
    constexpr int NQ = (G4 + 64 * NW - 1) / (64 * NW);
    float4 bq[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = tid + k * 64 * NW;
        const int co = n0 + (q % (BN / 4)) * 4;
        bq[k] = (a.ksplit == 1 && a.bias && q < G4 && co < a.Cout) ? *(const float4*)(a.bias + co)
                                                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();   // every wave is done with its buffer: the LDS holds the partial tiles

    // acc[i][n][r] = D[pixel 16i + 4(l>>4) + r][channel 16n + (l&15)], pixel = tile row * 32 + column
    float* red = (float*)smem;                   // [8 waves][64][80] fp32
    const int ecol = lane & 15;
    const int erow = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 5; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(wave * 64 + i * 16 + erow + r) * BN + n * 16 + ecol] = acc[i][n][r];
    __syncthreads();
    // sum the 8 partials in wave order, 4 channels of one pixel per thread and step
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int q = tid + k * 64 * NW;
        if (q >= G4) break;
        const int px = q / (BN / 4), c4 = (q - px * (BN / 4)) * 4;
        float4 v = *(const float4*)(red + px * BN + c4);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float4 u = *(const float4*)(red + (w * 64 + px) * BN + c4);
            v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
        }
        const int y = ty0 + (px >> 5), x = tx0 + (px & 31), co = n0 + c4;
        if (y < a.h && x < a.W && co < a.Cout) {
            const int64_t o = (((int64_t)bb * a.h + y) * a.W + x) * a.Cout + co;
            if (a.ksplit == 1) {
                if (a.bias) {
                    v.x += bq[k].x; v.y += bq[k].y; v.z += bq[k].z; v.w += bq[k].w;
                }
                if (a.res) {
                    const uint2 rv = *(const uint2*)(a.res + o);
                    v.x += __uint_as_float(rv.x << 16);
                    v.y += __uint_as_float(rv.x & 0xffff0000u);
                    v.z += __uint_as_float(rv.y << 16);
                    v.w += __uint_as_float(rv.y & 0xffff0000u);
                }
                uint2 ov;
                ov.x = pack_bf16x2(v.x, v.y);
                ov.y = pack_bf16x2(v.z, v.w);
                *(uint2*)(a.y + o) = ov;
            } else {
                *(float4*)(a.part + (int64_t)split * a.M * a.Cout + o) = v;
            }
        }
    }
}

// y[m][co] = bf16(bias[co] + sum_s part[s][m][co] (+ res[m][co])), summed in split order.  The
// splits are loaded 8 at a time, all in flight before any is added (a plain loop waits out
// every load).
__global__ __launch_bounds__(256) void conv_splitk_reduce_kernel(const float* __restrict__ part,
                                                                 const float* __restrict__ bias,
                                                                 const uint16_t* __restrict__ res,
                                                                 uint16_t* __restrict__ y, int64_t total4,
                                                                 int Cout, int ksplit) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i4 >= total4) return;
    const int64_t i = i4 * 4;
    float4 s = *(const float4*)(part + i);
    // 32-bit division when every element index fits (a uniform test)
    const int co = total4 <= 0x3fffffffLL ? (int)((uint32_t)i % (uint32_t)Cout) : (int)(i % Cout);
    const float4 bv = bias ? *(const float4*)(bias + co) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 1; k0 < ksplit; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < ksplit) v[u] = *(const float4*)(part + (int64_t)(k0 + u) * total4 * 4 + i);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (k0 + u < ksplit) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
    }
    if (bias) {
        s.x += bv.x;
        s.y += bv.y;
        s.z += bv.z;
        s.w += bv.w;
    }
    if (res) {
        const uint2 rv = *(const uint2*)(res + i);
        s.x += __uint_as_float(rv.x << 16);
        s.y += __uint_as_float(rv.x & 0xffff0000u);
        s.z += __uint_as_float(rv.y << 16);
        s.w += __uint_as_float(rv.y & 0xffff0000u);
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
                                                                 const float* __restrict__ res,
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
    if (res) acc += res[idx];
    y[idx] = acc;
}

}  // namespace

// Packed weights: chunk (co, ky, kx, c8) of 8 channels of w[Cout][3][3][Cin] goes to
// wp[ky][c8 / 4][kx][co][(c8 % 4) * 8 ..].  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void conv_pack_weights_kernel(const uint4* __restrict__ w, uint4* __restrict__ wp,
                                                                int Cin, int Cout) {
    const int64_t total = (int64_t)Cout * 9 * (Cin / 8);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int c8n = Cin / 8;
    const int c8 = (int)(i % c8n);
    const int64_t rest = i / c8n;               // (co * 3 + ky) * 3 + kx
    const int kx = (int)(rest % 3);
    const int ky = (int)((rest / 3) % 3);
    const int co = (int)(rest / 9);
    const int64_t o = ((((int64_t)ky * (Cin / 32) + c8 / 4) * 3 + kx) * Cout + co) * 4 + (c8 % 4);
    wp[o] = w[i];
}

ConvPlan plan_conv(const Geom& g, int Cout, bool bf16, bool gn_fused) {
    ConvPlan p{};
    if (!bf16) {
        p.kind = 0;
        return p;
    }
    const int ntx = (g.W + kTileTC - 1) / kTileTC;
    const int64_t big = (int64_t)g.B * ((g.h + 3) / 4) * ntx * ((Cout + 159) / 160);
    p.ktiles = 3 * g.C / 32;          // K stages (cc, ky)
    int ks = 1;
    const int64_t big8 = (int64_t)g.B * ((g.h + 7) / 8) * ntx * ((Cout + 159) / 160);
    if (gn_fused && big >= 384 && (big8 + 255) / 256 <= (big + 511) / 512) {
        // 256x160 tiles, one per CU, in no more rounds than the 128x160 tiles need at two per
        // CU: the tile the folded GroupNorm needs (its lanes and parameter table share the
        // workgroup's LDS).  Without a GroupNorm folded in, two 128x160 workgroups per CU
        // measured 2-5 % faster at every size tried (one workgroup's MFMAs fill the other's
        // barrier waits; same sums in the same order, so the outputs are bitwise equal).
        p.kind = 3;
        p.bm = 256;
        p.bn = 160;
        p.mtiles = (int)((int64_t)g.B * ((g.h + 7) / 8) * ntx);
        p.ntiles = (Cout + 159) / 160;
    } else if (big >= 384) {
        // enough 128x160 tiles for two per CU: shared ring, no K split
        p.kind = 1;
        p.bm = 128;
        p.bn = 160;
        p.mtiles = (int)((int64_t)g.B * ((g.h + 3) / 4) * ntx);
        p.ntiles = (Cout + 159) / 160;
    } else {
        // 64x80 tiles, K split over the 4 waves of a workgroup and across workgroups until
        // about 256 workgroups run, keeping >= 2 stages per wave
        p.kind = 2;
        p.bm = 64;
        p.bn = 80;
        p.mtiles = (int)((int64_t)g.B * ((g.h + 1) / 2) * ntx);
        p.ntiles = (Cout + 79) / 80;
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
    const int64_t M = (int64_t)g.B * g.h * g.W;
    p.ws_bytes = ks > 1 ? (size_t)ks * M * Cout * sizeof(float) : 0;
    return p;
}

hipError_t launch_conv_pack(int Cin, int Cout, const void* w, void* w_packed, hipStream_t stream) {
    const int64_t total = (int64_t)Cout * 9 * (Cin / 8);
    if (total == 0) return hipSuccess;
    if (!grid_fits((total + 255) / 256)) return hipErrorInvalidConfiguration;
    conv_pack_weights_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>((const uint4*)w, (uint4*)w_packed,
                                                                                Cin, Cout);
    return hipGetLastError();
}

namespace {

ConvArgs conv_args(const Geom& g, const ConvPlan& plan, int Cout, const void* x_patch, const void* x_stale,
                   const void* w, bool w_packed, const float* bias, const void* res, void* y, void* ws) {
    ConvArgs a{};
    a.xp = (const uint16_t*)x_patch;
    a.xs = (const uint16_t*)x_stale;
    a.w = (const uint16_t*)w;
    a.bias = bias;
    a.res = (const uint16_t*)res;
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
    a.ntx = (g.W + kTileTC - 1) / kTileTC;
    const int tr = plan.kind == 3 ? 8 : plan.kind == 1 ? 4 : 2;     // tile rows
    a.nty = (g.h + tr - 1) / tr;
    a.mtiles = plan.mtiles;
    a.ntiles = plan.ntiles;
    a.kstages = plan.ktiles;
    a.ksplit = plan.ksplit;
    a.wpacked = w_packed ? 1 : 0;
    return a;
}

}  // namespace

hipError_t launch_conv(const Geom& g, const ConvPlan& plan, bool bf16, int Cout, const void* x_patch,
                       const void* x_stale, const void* w, bool w_packed, const float* bias, const void* res,
                       void* y, void* ws, hipStream_t stream) {
    if (!bf16) {
        const int64_t total = (int64_t)g.B * g.h * g.W * Cout;
        const int64_t blocks = (total + 255) / 256;
        if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
        conv3x3_f32_direct_kernel<<<(unsigned)blocks, 256, 0, stream>>>(
            (const float*)x_patch, (const float*)x_stale, (const float*)w, bias, (const float*)res, (float*)y, g.B,
            g.H, g.W, g.C, Cout, g.h, g.r0);
        return hipGetLastError();
    }
    ConvArgs a = conv_args(g, plan, Cout, x_patch, x_stale, w, w_packed, bias, res, y, ws);
    const int64_t nwg = (int64_t)plan.mtiles * plan.ntiles * plan.ksplit;
    const int64_t total4 = (int64_t)a.M * Cout / 4;
    if (!grid_fits(nwg) || (plan.ksplit > 1 && !grid_fits((total4 + 255) / 256))) return hipErrorInvalidConfiguration;
    const unsigned grid = (unsigned)nwg;
    if (plan.kind == 3) return hipErrorInvalidValue;     // only with a GroupNorm folded in
    if (plan.kind == 1)
        conv3x3_bf16_halo_tile_kernel<<<grid, kThreads, 0, stream>>>(a);
    else
        conv3x3_bf16_halo_wave8_kernel<<<grid, 512, 0, stream>>>(a);
    if (plan.ksplit > 1) {
        conv_splitk_reduce_kernel<<<(unsigned)((total4 + 255) / 256), 256, 0, stream>>>(
            (const float*)ws, bias, (const uint16_t*)res, (uint16_t*)y, total4, Cout, plan.ksplit);
    }
    return hipGetLastError();
}

bool conv_gn_fusable(const Geom& g, const ConvPlan& cp, const GnPlan& gp, int G, bool bf16) {
    if (!bf16 || cp.kind != 3 || cp.ksplit != 1 || G < 1 || gp.threads < G) return false;
    const int lanes = gp.threads / G;            // the normalising kernel's lanes per group
    return lanes * G <= 512 && G <= 512 && gn_fuse_table_offset(lanes, G) + 8 * g.C <= kGnFuseLds;
}

hipError_t launch_conv_gn(const Geom& g, const ConvPlan& cp, const GnPlan& gp, int G, float eps, int mode, int act,
                          const void* x_patch, const float* stale_stats, const float* gamma, const float* beta,
                          float* fresh_stats_out, void* u_stale, int Cout, const void* w, bool w_packed,
                          const float* bias, const void* res, void* y, const void* gn_partials,
                          hipStream_t stream) {
    if (!conv_gn_fusable(g, cp, gp, G, true)) return hipErrorInvalidValue;
    ConvArgs a = conv_args(g, cp, Cout, x_patch, u_stale, w, w_packed, bias, res, y, nullptr);
    a.gn_part = (const float2*)gn_partials;
    a.gn_stale = mode == 1 ? nullptr : stale_stats;
    a.gn_gamma = gamma;
    a.gn_beta = beta;
    a.gn_fresh_out = fresh_stats_out;
    a.ystate = (uint16_t*)u_stale;
    a.gn_nblk = gp.nblk;
    a.gn_G = G;
    a.gn_lanes = gp.threads / G;
    a.gn_mode = mode;
    a.gn_silu = act == 1 ? 1 : 0;
    a.gn_P = g.P;
    a.gn_i = g.i;
    a.gn_inv_count = gn_inv_count(g, G);
    a.gn_eps = eps;
    const int64_t nwg = (int64_t)cp.mtiles * cp.ntiles;
    if (!grid_fits(nwg)) return hipErrorInvalidConfiguration;
    conv3x3_bf16_gn_tile8_kernel<<<(unsigned)nwg, 512, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dp
