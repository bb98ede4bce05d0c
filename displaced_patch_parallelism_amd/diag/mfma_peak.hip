// Diagnostic: sustained MFMA throughput on gfx950 with no memory traffic (shapes x waves per SIMD).
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_peak.hip -o mfma_peak
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(512) void k16(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[5];
  for (int i = 0; i < 4; ++i) for (int e = 0; e < 8; ++e) a[i][e] = (__bf16)(0.001f * (lane + i + e));
  for (int i = 0; i < 5; ++i) for (int e = 0; e < 8; ++e) b[i][e] = (__bf16)(0.001f * (lane - i + e));
  f32x4 acc[4][5];
  for (int i = 0; i < 4; ++i) for (int n = 0; n < 5; ++n) acc[i][n] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 5; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[n], acc[i][n], 0, 0, 0);
  }
  float s = 0; for (int i = 0; i < 4; ++i) for (int n = 0; n < 5; ++n) s += acc[i][n][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
__global__ __launch_bounds__(512) void k32(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[2], b[2];
  for (int i = 0; i < 2; ++i) for (int e = 0; e < 8; ++e) { a[i][e] = (__bf16)(0.001f * (lane + i + e)); b[i][e] = (__bf16)(0.001f * (lane - i + e)); }
  f32x16 acc[2][2];
  for (int i = 0; i < 2; ++i) for (int n = 0; n < 2; ++n) for (int e = 0; e < 16; ++e) acc[i][n][e] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 5; ++r)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[n], acc[i][n], 0, 0, 0);
  }
  float s = 0; for (int i = 0; i < 2; ++i) for (int n = 0; n < 2; ++n) s += acc[i][n][0];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
template <typename F>
void run(const char* name, F kern, int threads, int iters, double flops_per_wave_iter, float* out) {
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  kern<<<256, threads>>>(out, iters);
  hipEventRecord(a); kern<<<256, threads>>>(out, iters); hipEventRecord(b); hipEventSynchronize(b);
  float ms; hipEventElapsedTime(&ms, a, b);
  const double fl = 256.0 * (threads / 64) * iters * flops_per_wave_iter;
  printf("%-22s threads %3d: %8.1f us  %7.1f TFLOP/s (%.1f%% of 2516)\n", name, threads, ms * 1e3, fl / ms / 1e9, fl / ms / 1e9 / 25.16);
}
int main() {
  float* out; hipMalloc(&out, 256 * 512 * 4);
  run("16x16x32 x20 indep", k16, 256, 4000, 20 * 16384.0, out);
  run("16x16x32 x20 indep", k16, 512, 4000, 20 * 16384.0, out);
  run("32x32x16 x20 (4 acc)", k32, 256, 4000, 20 * 32768.0, out);
  run("32x32x16 x20 (4 acc)", k32, 512, 4000, 20 * 32768.0, out);
  printf("err=%s\n", hipGetErrorString(hipDeviceSynchronize()));
}
