// LDS bank-conflict probe for gfx950: one launch per (operation, lane-address pattern); each
// lane repeats ds_read_b128 / ds_read_b64 / ds_write_b128 at the pattern's address. Run under
// rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS and divide
// each dispatch's counters by SQ_INSTS_LDS.
//   hipcc -O2 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -o /tmp/ldsbank mamba_selective_scan_02_amd/probe/ldsbank.hip
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ int swz_new(int r, int c) { return c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1); }
__device__ int swz_old(int r, int c) { return c ^ ((r >> 2) & 3); }

// byte address (in a 64 KB window) for lane l under pattern p
__device__ uint32_t addr_of(int p, int l) {
  const int tl = l & 15, g = l >> 4;
  switch (p) {
    case 0: return l * 16;                                  // contiguous
    case 1: return l * 64;                                  // 64 B row stride, same slot
    case 2: return tl * 64 + swz_new(tl, g) * 16;           // 16 rows x 4 slots, new swizzle
    case 3: return tl * 64 + swz_old(tl, g) * 16;           // 16 rows x 4 slots, old swizzle
    case 4: return tl * 64 + g * 16;                        // 16 rows x 4 slots, no swizzle
    case 5: return tl * 128 + ((g ^ ((tl >> 1) & 7)) & 7) * 16;  // 128 B rows, 8-slot swizzle
    case 6: return l * 64 + swz_new(l, 0) * 16;             // 64 rows, one logical slot, new
    case 7: return l * 64 + swz_old(l, 0) * 16;             // 64 rows, one logical slot, old
    case 8: return (l & 7) * 16 + (l >> 3) * 256;           // 8 lanes contiguous per 256 B
    case 9: return (l & 15) * 16 + (l >> 4) * 1024;         // 16 lanes contiguous per 1 KB
    case 10: return ((l ^ (l >> 3)) & 7) * 16 + (l >> 3) * 128;   // 128 B per 8 lanes, permuted
    case 11: return l * 16 * 2;                             // 32 B stride
    case 12: return tl * 16 + g * 256;                      // 16 lanes x 16 B per 256 B
    case 13: return (l & 1) * 16;                           // broadcast-ish: 2 addresses
    case 14: return 0;                                      // all lanes same address
  }
  return 0;
}

template <int OP>
__global__ void probe(int p, int iters, float *out) {
  __shared__ __attribute__((aligned(16))) float lds[16384];
  for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = (float)i;
  __syncthreads();
  const uint32_t a = addr_of(p, threadIdx.x) + (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    if (OP == 0) {
      f4 v;
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
      acc += v.x + v.w;
    } else if (OP == 1) {
      f2 v;
      asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
      acc += v.x + v.y;
    } else {
      f4 v = {acc, 1.f, 2.f, 3.f};
      asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" :: "v"(a), "v"(v) : "memory");
      acc += 1.f;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

int main() {
  float *out;
  (void)hipMalloc(&out, 256 * 64 * sizeof(float));
  const int iters = 2000;
  for (int op = 0; op < 3; ++op)
    for (int p = 0; p < 15; ++p) {
      if (op == 0) hipLaunchKernelGGL(probe<0>, dim3(256), dim3(64), 0, 0, p, iters, out);
      if (op == 1) hipLaunchKernelGGL(probe<1>, dim3(256), dim3(64), 0, 0, p, iters, out);
      if (op == 2) hipLaunchKernelGGL(probe<2>, dim3(256), dim3(64), 0, 0, p, iters, out);
      (void)hipDeviceSynchronize();
      printf("op %d pattern %d done\n", op, p);
    }
  (void)hipFree(out);
  return 0;
}
