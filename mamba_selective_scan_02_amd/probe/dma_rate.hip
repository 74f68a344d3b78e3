// Load throughput per CU from an L2-resident 1 MB buffer: global_load_lds_dwordx4 (direct to
// LDS) against global_load_dwordx4 into VGPRs, 4 / 8 / 16 waves per CU.
//   hipcc -O2 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o /tmp/dma_rate mamba_selective_scan_02_amd/probe/dma_rate.hip && /tmp/dma_rate
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef __attribute__((ext_vector_type(4))) unsigned u4;

__global__ void dma_k(const unsigned *src, int iters, int span_kb, unsigned *out) {
  __shared__ __attribute__((aligned(16))) unsigned lds[8192];   // 32 KB
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t ldsb = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)&lds[wv * 256];
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(ldsb);
  for (int it = 0; it < iters; ++it) {
    const unsigned *p = src + ((blockIdx.x * 37 + it * 64 + wv * 16) % (span_kb * 4)) * 64 + lane * 4;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(p), "s"(m0v) : "memory", "m0");
    if ((it & 7) == 7) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  out[blockIdx.x * blockDim.x + threadIdx.x] = lds[threadIdx.x];
}
__global__ void vgpr_k(const unsigned *src, int iters, int span_kb, unsigned *out) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  u4 acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    const u4 *p = (const u4 *)(src + ((blockIdx.x * 37 + it * 64 + wv * 16) % (span_kb * 4)) * 64) + lane;
    u4 v = __builtin_nontemporal_load(p);
    acc ^= v;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
int main() {
  unsigned *src, *out;
  const int span_kb = 1024;    // 1 MB source, L2-resident
  (void)hipMalloc(&src, span_kb * 1024 + 4096); (void)hipMemset(src, 1, span_kb * 1024 + 4096);
  (void)hipMalloc(&out, 1 << 22);
  hipEvent_t e0, e1; (void)hipEventCreate(&e0); (void)hipEventCreate(&e1);
  const int iters = 2000;
  for (int kind = 0; kind < 2; ++kind)
    for (int wpw : {4, 8, 16}) {
      const int grid = 256, block = 64 * wpw;
      auto go = [&]() {
        if (kind == 0) hipLaunchKernelGGL(dma_k, dim3(grid), dim3(block), 0, 0, src, iters, span_kb, out);
        else hipLaunchKernelGGL(vgpr_k, dim3(grid), dim3(block), 0, 0, src, iters, span_kb, out);
      };
      go(); (void)hipDeviceSynchronize();
      (void)hipEventRecord(e0); go(); (void)hipEventRecord(e1); (void)hipEventSynchronize(e1);
      float ms; (void)hipEventElapsedTime(&ms, e0, e1);
      const double bytes = (double)grid * wpw * iters * 1024;
      printf("%s waves/CU %2d: %.3f ms  %.1f TB/s  %.1f B/clk/CU\n", kind == 0 ? "dma " : "vgpr", wpw, ms,
             bytes / (ms * 1e-3) / 1e12, bytes / (ms * 1e-3) / 2.4e9 / 256);
    }
  return 0;
}
