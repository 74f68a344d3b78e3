// bf16 MFMA throughput on gfx950: back-to-back v_mfma_f32_16x16x32_bf16 and 32x32x16_bf16 with
// 1 or 4 independent accumulators per wave at 1, 2 and 4 waves per SIMD. Prints cycles per
// MFMA per SIMD (2.4 GHz). The TFLOP/s column counts 2 flops per MAC with 16384 MACs per
// instruction, which is right for 32x32x16 and twice the true figure for 16x16x32 (8192 MACs).
//   hipcc -O2 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o /tmp/mfma_rate mamba_selective_scan_02_amd/probe/mfma_rate.hip && /tmp/mfma_rate
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

template <int NACC>
__global__ void k16(int iters, float *out) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(threadIdx.x * 0.001f + i); b[i] = (__bf16)(i * 0.5f); }
  f32x4 acc[NACC];
  for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
  for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
template <int NACC>
__global__ void k32(int iters, float *out) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(threadIdx.x * 0.001f + i); b[i] = (__bf16)(i * 0.5f); }
  f32x16 acc[NACC];
  for (int j = 0; j < NACC; ++j) for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
  for (int j = 0; j < NACC; ++j) s += acc[j][0] + acc[j][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}
int main() {
  float *out; (void)hipMalloc(&out, 1024 * 1024 * sizeof(float));
  hipEvent_t e0, e1; (void)hipEventCreate(&e0); (void)hipEventCreate(&e1);
  const int iters = 4000;
  int clk = 0; (void)hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, 0);
  for (int wps : {1, 2, 4}) {
    const int grid = 256 * wps, block = 256;   // 4 waves per WG -> wps waves per SIMD
    for (int kind = 0; kind < 4; ++kind) {
      auto launch = [&]() {
        if (kind == 0) hipLaunchKernelGGL(k16<1>, dim3(grid), dim3(block), 0, 0, iters, out);
        if (kind == 1) hipLaunchKernelGGL(k16<4>, dim3(grid), dim3(block), 0, 0, iters, out);
        if (kind == 2) hipLaunchKernelGGL(k32<1>, dim3(grid), dim3(block), 0, 0, iters, out);
        if (kind == 3) hipLaunchKernelGGL(k32<4>, dim3(grid), dim3(block), 0, 0, iters, out);
      };
      launch(); (void)hipDeviceSynchronize();
      (void)hipEventRecord(e0); launch(); (void)hipEventRecord(e1); (void)hipEventSynchronize(e1);
      float ms = 0; (void)hipEventElapsedTime(&ms, e0, e1);
      const int nacc = (kind == 1 || kind == 3) ? 4 : 1;
      const double mfmas = (double)grid * (block / 64) * iters * nacc;   // wave-level MFMAs
      const double flops = mfmas * 16384.0 * 2;   // both shapes: 16384 MACs per instruction
      const double simd_cycles = ms * 1e-3 * 2.4e9 * 1024;
      printf("waves/SIMD %d  %s nacc %d: %.3f ms  %.1f TFLOP/s  %.2f cycles/MFMA/SIMD\n", wps,
             kind < 2 ? "16x16x32" : "32x32x16", nacc, ms, flops / (ms * 1e-3) / 1e12, simd_cycles / mfmas);
    }
  }
  printf("clock attr %d kHz\n", clk);
  return 0;
}
