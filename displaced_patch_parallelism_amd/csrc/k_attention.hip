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
// queries (8 waves x 32); K/V tiles of 64 tokens are staged in LDS, K and V
// row-major.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so
// that lane l owns query l%32: the running offset and sum stay in the lane.
// Q stays exact (bf16 as given); the scale is applied with the offset by one
// fp32 FMA per score.  The offset follows the running maximum lazily: a
// 32-key half is exponentiated with the current offset and its probability
// sum checked; only a sum above 2^8 (or the first or a ragged tile) makes the
// half take the slow path that finds its maximum and moves the offset.
// P^T (bf16) feeds O^T = V^T P^T directly from registers; within each 16-key
// MFMA step the key order is permuted identically on both operands so the
// S^T accumulator layout needs no shuffle.  The tile loop is software-
// pipelined so that each wave's exponentials run between its own MFMAs.  The
// token loader picks the fresh or stale buffer per key row, so tiles may
// straddle the band edges.  When (query tiles x heads) cannot fill the GPU,
// keys are split and the partial (O, max, sum) are merged by a second kernel
// in split order.
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
constexpr float kLazyMax = 256.0f;  // 2^kLazy: a larger half-tile probability sum takes the slow path

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

// A 64-bit value the caller knows is the same in every lane, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// LDS accesses of the tile loop.  The compiler makes an LDS read that it cannot tell apart from
// the ring buffers being filled by direct-to-LDS loads wait for every such load in flight; the
// loop waits for its own loads explicitly (vmcnt, then the barrier), so its reads are written so
// that no such wait is added: the K fragments as plain loads from a 32-bit LDS address, the V^T
// fragments as asm that waits for its own reads only.
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }
__device__ __forceinline__ bf16x8 lds_ld128(uint32_t addr) { return *(lds_bf16x8*)(uintptr_t)addr; }

// The lane index, read so that the compiler cannot reuse an earlier copy: values derived from it on
// rare paths (straddling tiles, the ragged last tile, the epilogue) are formed where they are used
// instead of being kept, and spilled, across the tile loop.
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Workgroup barrier that waits only for the wave's LDS accesses: __syncthreads() would also wait
// for the direct-to-LDS loads still in flight into the other ring stages.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// V^T operand fragments of 16-key group U, by ds_read_b64_tr_b16: within a 16-lane group lane c
// receives element c%4 of the 8-byte reads of lanes c/4, c/4+4, c/4+8, c/4+12, so lane j reads
// key (j/4) of a 4-key group at 4 consecutive dims and each lane ends up holding one dim for 4
// keys.  Four reads (va, va + 1 KB: keys +0/+8 of dims 0..31; vb = va ^ 64: dims 32..63), waited
// for in the same asm block.
template <int U, int SO = 0>
__device__ __forceinline__ void lds_read_vt(uint32_t va, uint32_t vb, s16x4& r00, s16x4& r10, s16x4& r01,
                                            s16x4& r11) {
    static_assert(SO + U * 2048 + 1024 < 65536, "LDS offset field");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\tds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\tds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r00), "=&v"(r10), "=&v"(r01), "=&v"(r11)
        : "v"(va), "v"(vb), "i"(SO + U * 2048), "i"(SO + U * 2048 + 1024));
}

// ---------------------------------------------------------------------------
// bf16 flash attention, d = 64.  K and V tiles of 64 keys arrive by
// global_load_lds_dwordx4 in a STAGES-deep LDS ring (16 KB per stage, rows of
// 128 bytes, 16-byte chunk c of row r at slot c ^ (r & 7)); the loader picks
// the fresh patch or the stale map per key row.  S^T = K Q^T per wave (lane
// = query); the PV operand V^T is read with transposing LDS reads, so V stays
// row-major in LDS.
// ---------------------------------------------------------------------------
template <int STAGES, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_bf16_d64_kernel(AttnArgs a) {
    constexpr int STAGE = 16 * 1024;          // K tile 8 KB + V tile 8 KB
    constexpr int LOADS = 16 / WAVES;         // DMA loads (1 KB chunks) per wave per stage
    constexpr int QTW = 32 * WAVES;           // queries per workgroup
    static_assert(16 % WAVES == 0 && WAVES >= 2 && (8 % LOADS) == 0, "a wave's loads are all K or all V");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];
    // all arguments in SGPRs from the start: with them loaded lazily the kernel, at its VGPR
    // limit, kept reloading spilled values inside the tile loop
    args_in_sgprs(a);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hsel = lane >> 5;
    // Workgroups are dispatched round-robin over the 8 XCDs (workgroup w on XCD w % 8).  Give
    // XCD x a contiguous run of the order (head, key split, query tile), query tile fastest:
    // the workgroups resident on an XCD then stream the same keys and values through its L2.
    // Everything derived from the workgroup index is uniform: kept in scalar registers.
    const int total = gridDim.x;
    const int xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int lt = xcd * (total >> 3) + (xcd < (total & 7) ? xcd : (total & 7)) + within;
    const int qt = __builtin_amdgcn_readfirstlane(lt % a.qtiles);
    const int rest = __builtin_amdgcn_readfirstlane(lt / a.qtiles);
    const int split = __builtin_amdgcn_readfirstlane(rest % a.kvsplit);
    const int bh = __builtin_amdgcn_readfirstlane(rest / a.kvsplit);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.heads);
    const int e = bh - b * a.heads;
    const int myq = qt * QTW + wave * 32 + (lane & 31);
    const bool qvalid = myq < a.Nq;
    const int col0 = e * D;

    // Q as given (bf16, exact): the scores come out of the MFMAs unscaled and the scale
    // (times log2 e, for the base-2 exponential) is applied in fp32 with the offset, one FMA
    // per score, so no rounding is added to the inputs
    bf16x8 q0, q1, q2, q3;
    {
        uint4 r[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                      make_uint4(0, 0, 0, 0)};
        if (qvalid) {
            const uint16_t* qp = a.q + ((int64_t)b * a.Nq + myq) * a.C + col0 + hsel * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = *(const uint4*)(qp + 16 * j);
        }
        q0 = __builtin_bit_cast(bf16x8, r[0]);
        q1 = __builtin_bit_cast(bf16x8, r[1]);
        q2 = __builtin_bit_cast(bf16x8, r[2]);
        q3 = __builtin_bit_cast(bf16x8, r[3]);
    }
    const float sc = a.sc;

    const int t0 = (int)((int64_t)a.kv_tiles * split / a.kvsplit);
    const int t1 = (int)((int64_t)a.kv_tiles * (split + 1) / a.kvsplit);
    const int nt = t1 - t0;

    // DMA lanes: wave w issues chunks w*LOADS+j (0..7 K rows, 8..15 V rows), 8 rows of 128 B per
    // chunk, so a wave loads only K or only V.  A tile wholly inside the fresh band or wholly in
    // the stale map (all but at most two tiles per split) takes one wave-uniform base address
    // (scalar arithmetic) plus a 32-bit per-lane byte offset; a tile that straddles a band edge or
    // runs past the last key picks the buffer per row.
    const int sub = lane >> 3;
    const int slot = lane & 7;
    const uint16_t* zero = (const uint16_t*)g_attn_zero;
    const bool is_k = wave * LOADS < 8;
    const uint16_t* fresh_buf = is_k ? a.k : a.v;
    const uint16_t* stale_buf = is_k ? a.ks : a.vs;
    // The wave's chunk j covers rows row0 + 8 j (its chunks are consecutive), so chunk j is chunk
    // 0 moved by 8 j rows of the wave-uniform base: one 32-bit lane offset (row0 + sub, slot) for
    // all of them.
    const uint32_t loff0 = (uint32_t)((((wave * LOADS) & 7) * 8 + sub) * a.C + col0 + (slot ^ sub) * 8) * 2u;
    // token n of the band at fresh_tok + n (n in [band0, band0 + Nq)), of the map at stale_tok + n;
    // both wave-uniform, kept in scalar registers
    const uint64_t fresh_tok = uniform_u64((uint64_t)(fresh_buf + ((int64_t)b * a.Nq - a.band0) * a.C));
    const uint64_t stale_tok = uniform_u64((uint64_t)(stale_buf + (int64_t)b * a.N * a.C));
    const uint32_t row_bytes = (uint32_t)a.C * 2u;
#define DPA_ISSUE(T, BUF)                                                                           \
    do {                                                                                            \
        char* st_ = smem + (BUF) * STAGE;                                                           \
        const int n0_ = (T) * KT;                                                                   \
        const bool in_band_ = n0_ >= a.band0 && n0_ + KT <= a.band0 + a.Nq;                         \
        const bool in_stale_ = (n0_ + KT <= a.band0 || n0_ >= a.band0 + a.Nq) && n0_ + KT <= a.N;  \
        if (in_band_ || in_stale_) {                                                                \
            const char* base_ = (const char*)((in_band_ ? fresh_tok : stale_tok) +                  \
                                              (uint64_t)(uint32_t)n0_ * row_bytes);                 \
            _Pragma("unroll") for (int j = 0; j < LOADS; ++j)                                       \
                __builtin_amdgcn_global_load_lds((const void*)(base_ + (uint64_t)j * 8 * row_bytes + loff0), \
                                                 (lds_void*)(st_ + (wave * LOADS + j) * 1024), 16, 0, 0); \
        } else {                                                                                    \
            const int ln_ = lane_now();                                                             \
            _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                     \
                const int q_ = wave * LOADS + j;                                                    \
                const int row_ = (q_ & 7) * 8 + (ln_ >> 3);                                         \
                const int n_ = n0_ + row_;                                                          \
                const int ch_ = ((ln_ & 7) ^ (row_ & 7)) * 8;                                       \
                const uint16_t* g_ = n_ < a.N ? kv_row(fresh_buf, stale_buf, b, n_, a, col0 + ch_) : zero; \
                __builtin_amdgcn_global_load_lds((const void*)g_, (lds_void*)(st_ + q_ * 1024), 16, 0, 0); \
            }                                                                                       \
        }                                                                                           \
    } while (0)

    // K operand reads (A of S^T): key row kb*32 + (l & 31), 16-byte chunk (2 ks + hsel) ^ (row & 7)
    // for k-step ks, i.e. byte offset koff0 ^ (32 ks) (the XOR only flips bits 5..6)
    const int krow = lane & 31;
    const uint32_t koff0 = (uint32_t)(krow * 128 + ((hsel ^ (krow & 7)) * 16));
    // V^T operand reads: lane l = 16g + j reads key 16u + 4*(g>>1) + (j>>2) (+8 for the second
    // read) at dims 16*(g&1) + 4*(j&3) .. +3 (+32: chunk c + 4, i.e. byte offset ^ 64)
    uint32_t voff00;
    {
        const int gq = lane >> 4, jl = lane & 15;
        const int row = 4 * (gq >> 1) + (jl >> 2);
        const int d = 16 * (gq & 1) + 4 * (jl & 3);
        voff00 = (uint32_t)(8192 + row * 128 + (((d >> 3) ^ (row & 7)) * 16) + (d & 7) * 2);
    }

    // Online softmax with a lazily moved offset m (base-2 units of scale * score), kept negated
    // as nm_run: p = 2^(sc * s - m), the scale applied in fp32 by one FMA per score.  m is set to
    // the first half tile's maximum and moved up to the running maximum only when some score
    // exceeds it by more than kLazy (p <= 2^kLazy, harmless in the fp32 sums and the bf16 P);
    // since m is always a score that occurred, the largest p of a row is >= 1.
    f32x16 o0, o1;
    const f32x16 zacc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    o0 = zacc;
    o1 = zacc;
    float nm_run = 0.f;     // minus the offset
    float l_run = 0.f;
    bool first = true;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // lane offsets of the K fragments (k-steps 0..3: chunk (2 ks + hsel) ^ (row & 7), i.e. the
    // base XOR 32 ks) and of the V^T fragments; a ring stage is a constant offset added to them
    const uint32_t kl0 = lds_addr(smem) + koff0, kl1 = kl0 ^ 32u, kl2 = kl0 ^ 64u, kl3 = kl0 ^ 96u;
    const uint32_t vl0 = lds_addr(smem) + voff00, vl1 = vl0 ^ 64u;

    // Scores of the 32-key half KO / 4096 of the tile in ring stage SG.
#define DPA_S(S, SG, KO)                                                                            \
    do {                                                                                            \
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld128(kl0 + (SG) * STAGE + (KO)), q0, zacc, 0, 0, 0); \
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld128(kl1 + (SG) * STAGE + (KO)), q1, S, 0, 0, 0); \
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld128(kl2 + (SG) * STAGE + (KO)), q2, S, 0, 0, 0); \
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld128(kl3 + (SG) * STAGE + (KO)), q3, S, 0, 0, 0); \
    } while (0)
    // Probabilities of a half (P^T operands PA: keys 16u + 4*hsel + {0..3, 8..11} of its first 16,
    // PB: of its second 16) and their sum, in one chain; the row sum adds the same bf16 values
    // P.V uses.
#define DPA_EXP(S, PA, PB, L)                                                                       \
    do {                                                                                            \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) S[i] = __builtin_amdgcn_exp2f(fmaf(S[i], sc, nm_run)); \
        PA = pack_probs<0>(S);                                                                      \
        PB = pack_probs<2>(S);                                                                      \
        const uint4 wa_ = __builtin_bit_cast(uint4, PA), wb_ = __builtin_bit_cast(uint4, PB);       \
        float l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa_.x), ones, 0.f, false); \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa_.y), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa_.z), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa_.w), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wb_.x), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wb_.y), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wb_.z), ones, l_, false);   \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wb_.w), ones, l_, false);   \
        L = l_;                                                                                     \
    } while (0)
    // Slow path of a half of tile T (in ring stage SG): its raw scores again, keys >= N masked
    // (-inf, so p = 0), its maximum (both lane halves of a query), the offset moved if it is
    // exceeded by more than kLazy (everything accumulated so far rescaled), and the half
    // exponentiated again.
#define DPA_FIX(S, SG, KO, T, PA, PB, L)                                                            \
    do {                                                                                            \
        DPA_S(S, SG, KO);                                                                           \
        if (((T) + 1) * KT > a.N) {                                                                 \
            const int kvalid_ = a.N - ((T) * KT + 4 * (lane_now() >> 5)) - (KO) / 128;              \
            _Pragma("unroll") for (int i = 0; i < 16; ++i)                                          \
                if (8 * (i >> 2) + (i & 3) >= kvalid_) S[i] = -INFINITY;                            \
        }                                                                                           \
        float m0_ = fmaxf(S[0], S[1]), m1_ = fmaxf(S[2], S[3]);                                     \
        _Pragma("unroll") for (int i = 4; i < 16; i += 4) {                                         \
            m0_ = fmaxf(fmaxf(m0_, S[i]), S[i + 1]);                                                \
            m1_ = fmaxf(fmaxf(m1_, S[i + 2]), S[i + 3]);                                            \
        }                                                                                           \
        float mx_ = fmaxf(m0_, m1_) * sc;                                                           \
        mx_ = fmaxf(mx_, __shfl_xor(mx_, 32));                                                      \
        if (first || mx_ > -nm_run + kLazy) {                                                       \
            const float nmnew_ = first ? -mx_ : fminf(nm_run, -mx_);                                \
            const float alpha_ = first ? 1.f : __builtin_amdgcn_exp2f(nmnew_ - nm_run);             \
            l_run *= alpha_;                                                                        \
            o0 *= alpha_;                                                                           \
            o1 *= alpha_;                                                                           \
            nm_run = nmnew_;                                                                        \
        }                                                                                           \
        first = false;                                                                              \
        DPA_EXP(S, PA, PB, L);                                                                      \
    } while (0)
    // One slice of a half's softmax, placed after one MFMA: the exponentials of score pair J, the
    // bf16 pack of pair J-1 and the row-sum step of pair J-2 (the same operations, in the same
    // order, as DPA_EXP); the fence keeps the compiler from regrouping the slices.
#define DPA_SLICE(S, J)                                                                             \
    do {                                                                                            \
        S[2 * (J)] = __builtin_amdgcn_exp2f(fmaf(S[2 * (J)], sc, nm_run));                          \
        S[2 * (J) + 1] = __builtin_amdgcn_exp2f(fmaf(S[2 * (J) + 1], sc, nm_run));                  \
        if ((J) >= 1) w[(J) - 1] = pack_bf16x2(S[2 * (J) - 2], S[2 * (J) - 1]);                     \
        if ((J) == 2) l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0]), ones, 0.f, false); \
        if ((J) > 2) l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[(J) - 2]), ones, l_, false); \
        __builtin_amdgcn_sched_barrier(0);                                                          \
    } while (0)
#define DPA_VT(A, B) __builtin_bit_cast(bf16x8, __builtin_shufflevector(A, B, 0, 1, 2, 3, 4, 5, 6, 7))
    // One pipelined block: the scores N of half KO/4096 of the next tile (its K in ring stage SN)
    // and P.V of the current tile's 16-key groups U0, U1 (its V in stage SC; operands PIA, PIB),
    // alternating MFMA by MFMA with the softmax of the raw scores S (into POA, POB and the sum
    // L).  The stages are constants, so every LDS address is a lane offset plus an immediate.
#define DPA_BLOCK(N, SN, SC, KO, U0, U1, PIA, PIB, S, POA, POB, L)                                  \
    do {                                                                                            \
        uint32_t w[8];                                                                              \
        float l_ = 0.f;                                                                             \
        bf16x8 kf = lds_ld128(kl0 + (SN) * STAGE + (KO));                                           \
        s16x4 a0, b0, a1, b1;                                                                       \
        lds_read_vt<U0, (SC) * STAGE>(vl0, vl1, a0, b0, a1, b1);                                    \
        __builtin_amdgcn_sched_barrier(0);                                                          \
        N = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q0, zacc, 0, 0, 0);                         \
        kf = lds_ld128(kl1 + (SN) * STAGE + (KO));                                                  \
        DPA_SLICE(S, 0);                                                                            \
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(DPA_VT(a0, b0), PIA, o0, 0, 0, 0);             \
        DPA_SLICE(S, 1);                                                                            \
        N = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q1, N, 0, 0, 0);                            \
        kf = lds_ld128(kl2 + (SN) * STAGE + (KO));                                                  \
        DPA_SLICE(S, 2);                                                                            \
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(DPA_VT(a1, b1), PIA, o1, 0, 0, 0);             \
        lds_read_vt<U1, (SC) * STAGE>(vl0, vl1, a0, b0, a1, b1);                                    \
        DPA_SLICE(S, 3);                                                                            \
        N = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q2, N, 0, 0, 0);                            \
        kf = lds_ld128(kl3 + (SN) * STAGE + (KO));                                                  \
        DPA_SLICE(S, 4);                                                                            \
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(DPA_VT(a0, b0), PIB, o0, 0, 0, 0);             \
        DPA_SLICE(S, 5);                                                                            \
        N = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, q3, N, 0, 0, 0);                            \
        DPA_SLICE(S, 6);                                                                            \
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(DPA_VT(a1, b1), PIB, o1, 0, 0, 0);             \
        DPA_SLICE(S, 7);                                                                            \
        w[7] = pack_bf16x2(S[14], S[15]);                                                           \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[6]), ones, l_, false);    \
        l_ = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[7]), ones, l_, false);    \
        POA = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));                       \
        POB = __builtin_bit_cast(bf16x8, make_uint4(w[4], w[5], w[6], w[7]));                       \
        L = l_;                                                                                     \
    } while (0)

    // Software pipeline over the key tiles, so that a wave's exponentials run between its own
    // MFMAs (a SIMD does not overlap one wave's MFMAs with another wave's VALU work).  With
    // Sh(t) the scores of keys 32h.. of tile t and PVh(t) their P.V, iteration t runs
    //   block 1: S0(t+1) and PV0(t), with the softmax of S1(t); then the check of S1(t);
    //   block 2: S1(t+1) and PV1(t), with the softmax of S0(t+1); then the check of S0(t+1).
    // The ring then holds tile t (its V is still read), t+1 (its K is read), t+2 in flight, and
    // t+3 is requested into the stage t-1 left.  The last iteration computes S(t+1) from a stale
    // stage and discards it.
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nt) DPA_ISSUE(t0 + s, s);
    // Q is in registers before the loop (its loads were issued ahead of the first tiles')
    asm volatile("" ::"v"(q0), "v"(q1), "v"(q2), "v"(q3));
    if (nt >= 3) wait_vmcnt<2 * LOADS>();
    else if (nt == 2) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    ring_barrier();
    // A wave whose 32 queries all lie past the end of the patch (the last query tile of a band
    // that is not a multiple of the tile) computes nothing: it only keeps loading its share of
    // each tile and meets the workgroup at the same barriers, one per tile, leaving its SIMD's
    // issue slots to the other waves.
    if (qt * QTW + wave * 32 >= a.Nq) {
        for (int it = 0; it < nt; ++it) {
            if (it + 2 < nt) wait_vmcnt<LOADS>();
            else wait_vmcnt<0>();
            ring_barrier();
            if (it + 3 < nt) DPA_ISSUE(t0 + it + 3, (it + 3) & (STAGES - 1));
        }
        return;
    }
    f32x16 s1;          // raw S1 of the current tile
    bf16x8 p0, p1;      // P of the current tile's first half (its sum already in l_run)
    {
        f32x16 s0;
        DPA_S(s1, 0, 4096);
        float la;
        DPA_FIX(s0, 0, 0, t0, p0, p1, la);      // first tile: sets the offset
        l_run = la;
    }
    // one iteration with tile t in stage SC (its V read), tile t+1 in stage SN (its K read)
#define DPA_ITER(SC, SN, SI)                                                                        \
    if (it0 + (SC) < nt) {                                                                          \
        const int it = it0 + (SC);                                                                  \
        const int t = t0 + it;                                                                      \
        if (it + 2 < nt) wait_vmcnt<LOADS>();                                                       \
        else wait_vmcnt<0>();                                                                       \
        ring_barrier();                                                                             \
        if (it + 3 < nt) DPA_ISSUE(t + 3, SI);                                                      \
        f32x16 n0;                                                                                  \
        bf16x8 p2, p3;                                                                              \
        float lb;                                                                                   \
        DPA_BLOCK(n0, SN, SC, 0, 0, 1, p0, p1, s1, p2, p3, lb);                                     \
        if (__builtin_amdgcn_ballot_w64((t + 1) * KT > a.N || !(lb <= kLazyMax)))                   \
            DPA_FIX(s1, SC, 4096, t, p2, p3, lb);                                   \
        l_run += lb;                                                                                \
        float la;                                                                                   \
        DPA_BLOCK(s1, SN, SC, 4096, 2, 3, p2, p3, n0, p0, p1, la);                                  \
        if (it + 1 < nt) {                                                                          \
            if (__builtin_amdgcn_ballot_w64((t + 2) * KT > a.N || !(la <= kLazyMax)))               \
                DPA_FIX(n0, SN, 0, t + 1, p0, p1, la);                              \
            l_run += la;                                                                            \
        }                                                                                           \
    }
    static_assert(STAGES == 4, "the loop is unrolled by the ring depth");
    for (int it0 = 0; it0 < nt; it0 += STAGES) {
        DPA_ITER(0, 1, 3)
        DPA_ITER(1, 2, 0)
        DPA_ITER(2, 3, 1)
        DPA_ITER(3, 0, 2)
    }
#undef DPA_ITER
#undef DPA_BLOCK
#undef DPA_VT
#undef DPA_SLICE
#undef DPA_FIX
#undef DPA_EXP
#undef DPA_S
#undef DPA_ISSUE

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const int lne = lane_now();
    const int myq_e = qt * QTW + wave * 32 + (lne & 31), hsel_e = lne >> 5;
    if (myq_e >= a.Nq) return;
    // O^T layout: lane owns query myq_e, dims db*32 + 8q + 4*hsel_e + r
    if (a.kvsplit == 1) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = a.o + ((int64_t)b * a.Nq + myq_e) * a.C + col0 + 4 * hsel_e;
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
        const int64_t row = ((int64_t)split * a.B * a.heads + bh) * a.Nq + myq_e;
        float* prow = a.part_o + row * D + 4 * hsel_e;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *(float4*)(prow + 8 * q) = make_float4(o0[4 * q + 0], o0[4 * q + 1], o0[4 * q + 2], o0[4 * q + 3]);
            *(float4*)(prow + 32 + 8 * q) = make_float4(o1[4 * q + 0], o1[4 * q + 1], o1[4 * q + 2], o1[4 * q + 3]);
        }
        if (hsel_e == 0) a.part_ml[row] = make_float2(-nm_run, l_tot);
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
    // 32-bit division when every row index fits (a uniform test): the 64-bit one is a long
    // sequence ahead of the loads
    int q, bh;
    if (rows <= 0xffffffffLL) {
        q = (int)((uint32_t)row % (uint32_t)Nq);
        bh = (int)((uint32_t)row / (uint32_t)Nq);
    } else {
        q = (int)(row % Nq);
        bh = (int)(row / Nq);
    }
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
    // Pick the key split that fills whole rounds of workgroup slots best (>= 2 key tiles per
    // split), preferring fewer splits: fewer, longer workgroups pay the pipeline fill, the
    // partial write and the merge less often.  Two workgroups fit a CU (64 KB of LDS each), so a
    // grid of at least 512 workgroups runs in rounds of 512; a smaller one is counted in rounds
    // of 256 (one per CU: a CU's second workgroup would only share its SIMDs).  3840px layer: 290
    // units x 7 splits = 2030 workgroups, 99 % of four rounds of 512 (6 splits: 85 %).
    int ks = 1;
    double best = 0.0;
    for (int k = 1; k <= kMaxSplit; ++k) {
        if (k > 1 && kv_tiles / k < 2) break;
        const int64_t wgs = units * k;
        const int64_t slots = wgs >= 512 ? 512 : 256;
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
#define DP_F32_ATTN(HD)                                                                             \
    attn_f32_kernel<HD><<<blocks, 64, 0, stream>>>((const float*)q, (const float*)k, (const float*)v, \
                                                   (const float*)k_stale, (const float*)v_stale,    \
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
