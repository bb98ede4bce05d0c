// Band splice: stale[b, r0:r0+h] = x_patch[b], bit for bit.
//
// The fresh band of patch i becomes part of the resident stale map that the
// next denoising step reads as context (DistriFusion summary on
// atlas.scime.ai, Approach; study.space page, Method).  In NHWC with row
// bands, batch b's band is one contiguous span, so the splice is B
// contiguous copies.  HBM-bound: each byte is read once and written once.
// 16-byte vector accesses, four in flight per thread, one batch per
// blockIdx.y; a scalar tail covers spans that are not a multiple of 16 bytes.

#include "dp_device.h"
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void band_copy16_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst, int64_t n16,
                                                               int64_t src_stride16, int64_t dst_stride16) {
    const u32x4* s = src + (int64_t)blockIdx.y * src_stride16;
    u32x4* d = dst + (int64_t)blockIdx.y * dst_stride16;
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
        const int64_t idx = base + j * kThreads;
        if (idx < n16) v[j] = __builtin_nontemporal_load(s + idx);
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
        const int64_t idx = base + j * kThreads;
        if (idx < n16) __builtin_nontemporal_store(v[j], d + idx);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void band_copy_elem_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                                  int64_t n, int64_t src_stride,
                                                                  int64_t dst_stride) {
    const T* s = src + (int64_t)blockIdx.y * src_stride;
    T* d = dst + (int64_t)blockIdx.y * dst_stride;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * kThreads)
        d[idx] = s[idx];
}

}  // namespace

hipError_t launch_band_copy(const void* src, void* dst, const Geom& g, size_t es, hipStream_t stream) {
    const int64_t band_elems = g.band_tokens() * g.C;   // per batch
    const int64_t map_elems = g.map_tokens() * g.C;
    char* dst_band = (char*)dst + (size_t)g.r0 * g.W * g.C * es;
    const size_t band_bytes = (size_t)band_elems * es;
    const size_t map_bytes = (size_t)map_elems * es;
    const bool vec_ok = band_bytes % 16 == 0 && map_bytes % 16 == 0 && ((uintptr_t)dst_band & 15u) == 0 &&
                        ((uintptr_t)src & 15u) == 0;
    if (vec_ok) {
        const int64_t n16 = (int64_t)(band_bytes / 16);
        dim3 grid((unsigned)((n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll)), (unsigned)g.B);
        if (n16 == 0) return hipSuccess;
        band_copy16_kernel<<<grid, kThreads, 0, stream>>>((const u32x4*)src, (u32x4*)dst_band, n16,
                                                         (int64_t)(band_bytes / 16), (int64_t)(map_bytes / 16));
    } else {
        const int64_t blocks = (band_elems + kThreads - 1) / kThreads;
        dim3 grid((unsigned)(blocks < 4096 ? blocks : 4096), (unsigned)g.B);
        if (es == 2)
            band_copy_elem_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(
                (const uint16_t*)src, (uint16_t*)dst_band, band_elems, band_elems, map_elems);
        else
            band_copy_elem_kernel<uint32_t><<<grid, kThreads, 0, stream>>>(
                (const uint32_t*)src, (uint32_t*)dst_band, band_elems, band_elems, map_elems);
    }
    return hipGetLastError();
}

}  // namespace dp
