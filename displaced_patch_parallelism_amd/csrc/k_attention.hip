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
// base-2 domain (log2(e) folded into the scale).  A workgroup holds 256
// queries (8 waves x 32); K/V tiles of 64 tokens are staged in LDS, K
// row-major and V transposed.  Each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so that lane l owns query l%32: the running
// offset and sum stay in the lane.  Q is pre-scaled and the S MFMAs start
// from C = -offset, so S - offset comes out of the MFMA; the offset follows
// the running maximum lazily (the cross-half exchange happens only when it
// moves).
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
constexpr int KT = 64;          // keys per tile
constexpr int kStages = 4;      // LDS ring depth (16 KB per stage)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;
constexpr float kLazy = 8.0f;     // offset moves when a score exceeds it by more than this (log2)

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
    int qtiles;        // query tiles per (batch, head)
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

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((vector_size(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __attribute__((aligned(64))) uint4 g_attn_zero[8];   // never written: a zero key/value row

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 4 bf16 of V^T for the PV operand via the transposing LDS read (see the lane map below).
__device__ __forceinline__ s16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// ---------------------------------------------------------------------------
// bf16 flash attention, d = 64.  K and V tiles of 64 keys arrive by
// global_load_lds_dwordx4 in a STAGES-deep LDS ring (16 KB per stage, rows of
// 128 bytes, 16-byte chunk c of row r at slot c ^ (r & 7)); the loader picks
// the fresh patch or the stale map per key row.  S^T = K Q^T per wave (lane
// = query).  The PV operand V^T is read with ds_read_b64_tr_b16: within a
// 16-lane group, lane c receives element c%4 of the 8-byte reads of lanes
// c/4, c/4+4, c/4+8, c/4+12, so lane j reads key (j/4) of a 4-key group at
// dims 4*(j%4)..+3 and each lane ends up holding one dim for 4 keys -- V
// stays row-major in LDS.
// ---------------------------------------------------------------------------
template <int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_bf16_d64_kernel(AttnArgs a) {
    constexpr int STAGE = 16 * 1024;          // K tile 8 KB + V tile 8 KB
    constexpr int LOADS = 16 / WAVES;         // DMA loads (1 KB chunks) per wave per stage
    constexpr int QTW = 32 * WAVES;           // queries per workgroup
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
    // all arguments in SGPRs from the start: with them loaded lazily the kernel, at its VGPR
    // limit, kept reloading spilled values inside the tile loop
    args_in_sgprs(a);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hsel = lane >> 5;
    // Workgroups are dispatched round-robin over the 8 XCDs (workgroup w on XCD w % 8).  Give
    // XCD x a contiguous run of the order (head, key split, query tile), query tile fastest:
    // the workgroups resident on an XCD then stream the same keys and values through its L2.
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int lt = xcd * (total >> 3) + (xcd < (total & 7) ? xcd : (total & 7)) + within;
    const int qt = lt % a.qtiles;
    const int rest = lt / a.qtiles;
    const int split = rest % a.kvsplit;
    const int bh = rest / a.kvsplit;
    const int b = bh / a.heads;
    const int e = bh - b * a.heads;
    const int myq = qt * QTW + wave * 32 + (lane & 31);
    const bool qvalid = myq < a.Nq;
    const int col0 = e * D;

    // Q scaled by scale * log2(e) once (rounded to bf16), so S = K Q^T is already in the
    // base-2 exponent domain
    bf16x8 q0, q1, q2, q3;
    {
        uint4 r[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                      make_uint4(0, 0, 0, 0)};
        if (qvalid) {
            const uint16_t* qp = a.q + ((int64_t)b * a.Nq + myq) * a.C + col0 + hsel * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = *(const uint4*)(qp + 16 * j);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float f[8];
            unpack8(r[j], f);
#pragma unroll
            for (int u = 0; u < 8; ++u) f[u] *= a.sc;
            r[j] = pack8(f);
        }
        q0 = __builtin_bit_cast(bf16x8, r[0]);
        q1 = __builtin_bit_cast(bf16x8, r[1]);
        q2 = __builtin_bit_cast(bf16x8, r[2]);
        q3 = __builtin_bit_cast(bf16x8, r[3]);
    }

    const int t0 = (int)((int64_t)a.kv_tiles * split / a.kvsplit);
    const int t1 = (int)((int64_t)a.kv_tiles * (split + 1) / a.kvsplit);
    const int nt = t1 - t0;

    // DMA lanes: wave w issues chunks w*LOADS+j (0..7 K rows, 8..15 V rows), 8 rows of 128 B per chunk.
    // A tile wholly inside the fresh band or wholly in the stale map (all but at most two tiles
    // per split) takes one wave-uniform base pointer plus a fixed per-lane offset; a tile that
    // straddles a band edge or runs past the last key picks the buffer per row.
    const int sub = lane >> 3;
    const int slot = lane & 7;
    const uint16_t* zero = (const uint16_t*)g_attn_zero;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int loff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int row = ((wave_u * LOADS + j) & 7) * 8 + sub;
        loff[j] = row * a.C + col0 + (slot ^ (row & 7)) * 8;
    }
    const int64_t fresh_base = (int64_t)b * a.Nq - a.band0;   // token n of the band at fresh_base + n
    const int64_t stale_base = (int64_t)b * a.N;
#define DPA_ISSUE(T, BUF)                                                                           \
    do {                                                                                            \
        char* st_ = smem + (BUF) * STAGE;                                                           \
        const int n0_ = (T) * KT;                                                                   \
        const bool in_band_ = n0_ >= a.band0 && n0_ + KT <= a.band0 + a.Nq;                         \
        const bool in_stale_ = (n0_ + KT <= a.band0 || n0_ >= a.band0 + a.Nq) && n0_ + KT <= a.N;  \
        if (in_band_ || in_stale_) {                                                                \
            _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                     \
                const int q_ = wave_u * LOADS + j;                                                  \
                const uint16_t* buf_ = in_band_ ? (q_ < 8 ? a.k : a.v) : (q_ < 8 ? a.ks : a.vs);    \
                const uint16_t* g_ = buf_ + ((in_band_ ? fresh_base : stale_base) + n0_) * a.C + loff[j]; \
                __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + q_ * 1024), 16, 0, 0); \
            }                                                                                       \
        } else {                                                                                    \
            _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                     \
                const int q_ = wave_u * LOADS + j;                                                  \
                const int row_ = (q_ & 7) * 8 + sub;                                                \
                const int n_ = n0_ + row_;                                                          \
                const int ch_ = (slot ^ (row_ & 7)) * 8;                                            \
                const uint16_t* fr_ = q_ < 8 ? a.k : a.v;                                           \
                const uint16_t* sl_ = q_ < 8 ? a.ks : a.vs;                                         \
                const uint16_t* g_ = n_ < a.N ? kv_row(fr_, sl_, b, n_, a, col0 + ch_) : zero;      \
                __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + q_ * 1024), 16, 0, 0); \
            }                                                                                       \
        }                                                                                           \
    } while (0)

    // K operand reads (A of S^T): key row kb*32 + (l & 31), 16-byte chunk 2*ks + hsel
    const int krow = lane & 31;
    int koff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = krow * 128 + (((2 * ks + hsel) ^ (krow & 7)) * 16);
    // V^T operand reads via tr reads: lane l = 16g + j; key 16u + 4*(g>>1) + 8h + (j>>2),
    // dims 32*db + 16*(g&1) + 4*(j&3) .. +3
    const int gq = lane >> 4, jl = lane & 15;
    int voff[2][2];   // [h][db] byte offsets inside the V tile for u = 0
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
            const int row = 4 * (gq >> 1) + 8 * h + (jl >> 2);          // + 16u (u*16 rows keeps row & 7)
            const int d = 32 * db + 16 * (gq & 1) + 4 * (jl & 3);
            voff[h][db] = 8192 + row * 128 + (((d >> 3) ^ (row & 7)) * 16) + (d & 7) * 2;
        }

    // Online softmax with a lazily moved offset: the QK MFMAs start from C = -m_run, so they
    // produce S - m_run directly and the exponent needs no subtraction.  m_run is set to the
    // first tile's maximum and moved up to the running maximum only when some score exceeds
    // it by more than kLazy (p <= 2^kLazy, harmless in fp32 sums and bf16 P); since m_run is
    // always a score that occurred, the largest p of a row is >= 1.
    f32x16 o0, o1, negm;
#pragma unroll
    for (int i = 0; i < 16; ++i) o0[i] = o1[i] = negm[i] = 0.f;
    float m_run = 0.f;
    float l_run = 0.f;
    bool first = true;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    if (nt > 0) {
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nt) DPA_ISSUE(t0 + s, s);
    }
    for (int it = 0; it < nt; ++it) {
        const int t = t0 + it;
        const int ahead = nt - 1 - it;
        if (STAGES >= 4 && ahead >= 2) wait_vmcnt<2 * LOADS>();
        else if (STAGES >= 3 && ahead >= 1) wait_vmcnt<LOADS>();
        else wait_vmcnt<0>();
        __syncthreads();
        const char* st = smem + (it % STAGES) * STAGE;

        // S^T[key][query], keys kb*32 + 8q + 4*hsel + r in s_kb[4q + r]
        f32x16 s0, s1;
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + koff[0]), q0, negm, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + 4096 + koff[0]), q0, negm, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + koff[1]), q1, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + 4096 + koff[1]), q1, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + koff[2]), q2, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + 4096 + koff[2]), q2, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + koff[3]), q3, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(st + 4096 + koff[3]), q3, s1, 0, 0, 0);

        // keys >= N occur only in a ragged last tile: excluded from the max, p = 0
        if ((t + 1) * KT > a.N) {
            const int kvalid = a.N - (t * KT + 4 * hsel);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 8 * (i >> 2) + (i & 3);
                if (off >= kvalid) s0[i] = -INFINITY;
                if (off + 32 >= kvalid) s1[i] = -INFINITY;
            }
        }
        // Exponentials against the current offset; the tile maximum (two independent chains of
        // 3-input maxima, v_max3_f32, over this lane's half of the keys) only decides whether
        // the offset must move, which is rare after the first tile: then the exponentials are
        // taken from the kept scores against the moved offset instead.
        f32x16 p0f, p1f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p0f[i] = __builtin_amdgcn_exp2f(s0[i]);
            p1f[i] = __builtin_amdgcn_exp2f(s1[i]);
        }
        float mx0 = fmaxf(s0[0], s0[1]), mx1 = fmaxf(s1[0], s1[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
            mx0 = fmaxf(fmaxf(mx0, s0[i]), s0[i + 1]);
            mx1 = fmaxf(fmaxf(mx1, s1[i]), s1[i + 1]);
        }
        float mx = fmaxf(mx0, mx1);
        if (__builtin_amdgcn_ballot_w64(first || mx > kLazy)) {
            mx = fmaxf(mx, __shfl_xor(mx, 32));     // max of S - m_run over the tile's keys
            const float delta = first ? mx : fmaxf(mx, 0.f);
            const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta);
            l_run *= alpha;
            o0 *= alpha;
            o1 *= alpha;
            m_run += delta;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p0f[i] = __builtin_amdgcn_exp2f(s0[i] - delta);
                p1f[i] = __builtin_amdgcn_exp2f(s1[i] - delta);
                negm[i] = -m_run;
            }
            first = false;
        }
        s0 = p0f;
        s1 = p1f;
        // P^T operands (keys 16u + 4*hsel + {0..3, 8..11}); the row sum adds the same bf16 values
        const bf16x8 p0 = pack_probs<0>(s0);
        const bf16x8 p1 = pack_probs<2>(s0);
        const bf16x8 p2 = pack_probs<0>(s1);
        const bf16x8 p3 = pack_probs<2>(s1);
#define DPA_SUM(PV)                                                                                 \
    do {                                                                                            \
        const uint4 w_ = __builtin_bit_cast(uint4, PV);                                             \
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w_.x), ones, l_run, false); \
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w_.y), ones, l_run, false); \
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w_.z), ones, l_run, false); \
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w_.w), ones, l_run, false); \
    } while (0)
        DPA_SUM(p0);
        DPA_SUM(p1);
        DPA_SUM(p2);
        DPA_SUM(p3);
#undef DPA_SUM
#define DPA_PV(U, PU)                                                                               \
    do {                                                                                            \
        const char* vb_ = st + (U) * 16 * 128;                                                      \
        const s16x4 a0_ = tr_read(vb_ + voff[0][0]);                                                \
        const s16x4 b0_ = tr_read(vb_ + voff[1][0]);                                                \
        const s16x4 a1_ = tr_read(vb_ + voff[0][1]);                                                \
        const s16x4 b1_ = tr_read(vb_ + voff[1][1]);                                                \
        const bf16x8 v0_ = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0_, b0_, 0, 1, 2, 3, 4, 5, 6, 7)); \
        const bf16x8 v1_ = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a1_, b1_, 0, 1, 2, 3, 4, 5, 6, 7)); \
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0_, PU, o0, 0, 0, 0);                          \
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1_, PU, o1, 0, 0, 0);                          \
    } while (0)
        DPA_PV(0, p0);
        DPA_PV(1, p1);
        DPA_PV(2, p2);
        DPA_PV(3, p3);
#undef DPA_PV
        // Tile t+3 goes into the stage tile t-1 left (every wave passed this iteration's barrier
        // after its last read of it).  Issued after this tile's V^T reads: the compiler makes the
        // transposing LDS reads wait for every direct-to-LDS load in flight, so loads issued
        // earlier in the iteration would be waited for here.
        if (it + STAGES - 1 < nt) DPA_ISSUE(t + STAGES - 1, (it + STAGES - 1) % STAGES);
    }
#undef DPA_ISSUE

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

// Merge of key-split partials, in split order.  One thread per (b*heads, query, 4 dims); all
// of a thread's partial loads are issued before any is used (kvsplit <= kMaxSplit).
constexpr int kMaxSplit = 16;

__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         uint16_t* __restrict__ o, int B, int heads, int C,
                                                         int Nq, int kvsplit) {
    params_in_sgprs(part_o, part_ml, o, B, heads, C, Nq, kvsplit);
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)B * heads * Nq;
    if (idx >= rows * (D / 4)) return;
    const int d4 = (int)(idx % (D / 4));
    const int64_t row = idx / (D / 4);  // (bh, q)
    const int q = (int)(row % Nq);
    const int bh = (int)(row / Nq);
    float2 ml[kMaxSplit];
    float4 v[kMaxSplit];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
        if (s < kvsplit) {
            ml[s] = part_ml[(int64_t)s * rows + row];
            v[s] = *(const float4*)(part_o + ((int64_t)s * rows + row) * D + d4 * 4);
        }
    }
    float M = kNegBig;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s)
        if (s < kvsplit) M = fmaxf(M, ml[s].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
        if (s < kvsplit) {
            const float w = __builtin_amdgcn_exp2f(ml[s].x - M);
            L = fmaf(ml[s].y, w, L);
            acc.x = fmaf(v[s].x, w, acc.x);
            acc.y = fmaf(v[s].y, w, acc.y);
            acc.z = fmaf(v[s].z, w, acc.z);
            acc.w = fmaf(v[s].w, w, acc.w);
        }
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
    const int64_t Nq = g.band_tokens();
    // 8 waves (256 queries) share each K/V tile.  A wave's tile loop is a serial chain (S
    // MFMAs, max, exponentials, P.V MFMAs), so throughput needs several waves per SIMD; the
    // 64 KB ring allows two workgroups per CU, i.e. four waves per SIMD.  Measured on
    // the small bands too (1024 and 128 queries), 8-wave tiles beat 4-wave ones.
    p.qtile = 256;
    p.qtiles = (int)((Nq + p.qtile - 1) / p.qtile);
    const int kv_tiles = (int)((g.map_tokens() + KT - 1) / KT);
    const int64_t units = (int64_t)p.qtiles * g.B * heads;
    // Pick the key split that fills whole rounds of 256 workgroups best (>= 2 key tiles per
    // split), preferring fewer splits: fewer, longer workgroups pay the pipeline fill, the
    // partial write and the merge less often.
    const int64_t slots = 256;
    int ks = 1;
    double best = 0.0;
    for (int k = 1; k <= kMaxSplit; ++k) {
        if (k > 1 && kv_tiles / k < 2) break;
        const int64_t wgs = units * k;
        const int64_t rounds = (wgs + slots - 1) / slots;
        const double eff = (double)wgs / (double)(rounds * slots);
        if (eff > best + 0.04) {
            best = eff;
            ks = k;
        }
    }
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
        if (!grid_fits((total + 63) / 64)) return hipErrorInvalidConfiguration;
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
    a.qtiles = plan.qtiles;
    const int64_t nwg = (int64_t)plan.qtiles * g.B * heads * plan.kvsplit;
    const int64_t merge_threads = (int64_t)g.B * heads * Nq * (D / 4);
    if (!grid_fits(nwg) || !grid_fits((merge_threads + 255) / 256)) return hipErrorInvalidConfiguration;
    const unsigned grid = (unsigned)nwg;
    attn_bf16_d64_kernel<kStages, 8><<<grid, 512, 0, stream>>>(a);
    if (plan.kvsplit > 1) {
        attn_merge_kernel<<<(unsigned)((merge_threads + 255) / 256), 256, 0, stream>>>(
            a.part_o, a.part_ml, (uint16_t*)o, g.B, heads, g.C, Nq, plan.kvsplit);
    }
    return hipGetLastError();
}

}  // namespace dp
