// LDS read bandwidth per CU: eight independent conflict-free ds_read_b128 (1 KB per wave each)
// per iteration, 4 / 8 / 16 waves per CU.
//   hipcc -O2 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o /tmp/lds_bw mamba_selective_scan_02_amd/probe/lds_bw.hip && /tmp/lds_bw
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef float f4 __attribute__((ext_vector_type(4)));
__global__ void k(int iters, float *out) {
  __shared__ __attribute__((aligned(16))) float lds[16384];   // 64 KB
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = (float)i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds + lane * 16;
  f4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    f4 v0, v1, v2, v3, v4, v5, v6, v7;
    const uint32_t a = base + ((it * 8 + wv) & 7) * 8192;
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\tds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
                 "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\tds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7) : "v"(a) : "memory");
    acc += v0 + v1 + v2 + v3 + v4 + v5 + v6 + v7;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}
int main() {
  float *out; (void)hipMalloc(&out, 1 << 22);
  hipEvent_t e0, e1; (void)hipEventCreate(&e0); (void)hipEventCreate(&e1);
  const int iters = 4000;
  for (int wpw : {4, 8, 16}) {
    const int grid = 256, block = 64 * wpw;
    hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, 0, iters, out); (void)hipDeviceSynchronize();
    (void)hipEventRecord(e0); hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, 0, iters, out);
    (void)hipEventRecord(e1); (void)hipEventSynchronize(e1);
    float ms; (void)hipEventElapsedTime(&ms, e0, e1);
    const double bytes = (double)grid * wpw * iters * 8 * 1024;
    printf("waves/CU %2d: %.3f ms  %.1f B/clk/CU\n", wpw, ms, bytes / (ms * 1e-3) / 2.4e9 / 256);
  }
  return 0;
}
