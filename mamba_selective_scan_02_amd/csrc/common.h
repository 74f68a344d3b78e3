// Shared device/host helpers of the gfx950 mixer library (internal; not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

typedef uint16_t bf16_t;  // bfloat16 bits

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- element conversion
__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
// round-to-nearest-even (lowers to v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}
// two floats to a bf16 pair (lo in the low half), both rounded to nearest even by one
// v_cvt_pk_bf16_f32 (the same rounding as f2bf)
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
// split-precision pair: hi = (bf16(u0), bf16(u1)), lo = (bf16(u0 - hi0), bf16(u1 - hi1)), the
// high parts widened back by shifting / masking their packed halves
__device__ __forceinline__ void split_bf2(float u0, float u1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf2(u0, u1);
  lo = pack_bf2(u0 - __uint_as_float(hi << 16), u1 - __uint_as_float(hi & 0xffff0000u));
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float *p) { return *p; }
  static __device__ __forceinline__ void st(float *p, float v) { *p = v; }
  static __device__ __forceinline__ float cvt(float v) { return v; }
};
template <> struct io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t *p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t *p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float cvt(bf16_t v) { return bf2f(v); }
};

// ---------------------------------------------------------------- math
// exp via the hardware base-2 exponential (v_exp_f32)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// SiLU(v) = v / (1 + e^-v); e^-v overflowing to +inf gives v * 0 = -0 for very negative v.
__device__ __forceinline__ float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-v * kLog2e));
}
// expm1(x) = e^x - 1 without cancellation: e^x - 1 from the hardware exp when |x| > 0.5
// (relative error ~2 ulp there), else the Taylor series to x^8 in Horner form (truncation
// below |x|^9 / 9! < 6e-9 relative for |x| <= 0.5).
__device__ __forceinline__ float expm1_f(float x) {
  if (fabsf(x) > 0.5f) return exp2_hw(x * kLog2e) - 1.0f;
  float r = __builtin_fmaf(x, 1.0f / 8.0f, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 7.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 6.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 5.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 4.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 3.0f), r, 1.0f);
  r = __builtin_fmaf(x * 0.5f, r, 1.0f);
  return x * r;
}
// softplus(v) = log(1 + e^v) from the hardware exp2 / log2: above 20 it equals v to within
// 2e-9 relative; otherwise e = e^v, w = 1 + e (rounded) and log(1 + e) = log(w) * e / (w - 1)
// (Goldberg's log1p method, "What every computer scientist should know about floating-point
// arithmetic", 1991), which cancels the rounding of w to first order (and is e itself when w
// rounds to 1).
__device__ __forceinline__ float softplus_f(float v) {
  if (v > 20.0f) return v;
  const float e = exp2_hw(v * kLog2e);
  const float w = 1.0f + e;
  if (w == 1.0f) return e;
  return __builtin_amdgcn_logf(w) * 0.69314718055994531f * (e * __builtin_amdgcn_rcpf(w - 1.0f));
}
// softplus_f without branches (dt_proj's epilogue, on its own or fused into the scan). With
// e = e^v and w = 1 + e rounded, delta = (w - 1) - e is that rounding exactly (w - 1 is exact),
// so log(1 + e) = log(w - delta) = log(w) - delta / w to within delta^2 / w^2 < 2^-48. 1 / w is
// taken as 2 - w (exact to second order in w - 1, where the correction matters) and as 0 once
// w >= 2 (there |delta| / w <= 2^-24 of log(w) >= log 2). Where 1 + e rounds to 1 this gives
// e itself (delta = -e). Above 20, v (within 2e-9 relative). One transcendental fewer than
// Goldberg's form log(w) e / (w - 1) of softplus_f.
__device__ __forceinline__ float softplus_sel(float v) {
  const float e = exp2_hw(v * kLog2e);
  const float w = 1.0f + e;
  const float delta = (w - 1.0f) - e;
  const float r = __builtin_fmaf(-delta, fmaxf(2.0f - w, 0.0f),
                                 __builtin_amdgcn_logf(w) * 0.69314718055994531f);
  return v > 20.0f ? v : r;
}

// Wait until every vector-memory operation of this wave has completed, without waiting on the
// LDS/scalar or export counters. (Stores and direct-to-LDS loads need not retire in issue order,
// so a partial vmcnt wait cannot prove a staged tile has landed.)
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
}
// At most N of this wave's vector-memory loads still in flight (the oldest ones complete
// first). Only for waves whose outstanding vector-memory operations are all loads: stores
// and loads do not retire in a common order.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes complete, then all
// waves meet. Global stores and direct-to-LDS prefetches issued before it stay in flight (a
// __syncthreads() would drain them); a prefetch that other waves read after a barrier must be
// waited for explicitly (wait_vmem_all / wait_vmem_le) before it. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-to-LDS 16-byte load issued opaquely: lane i of the wave writes bytes
// [lds_base + 16 i, +16) of LDS from its own global address. The compiler does not see the LDS
// write, so it inserts no waits for it; the caller synchronises (a vmcnt wait + barrier) before
// any wave reads that LDS. lds_base must be wave-uniform. No VGPR is written by the load.
__device__ __forceinline__ void dma16_opaque(const void *gptr, uint32_t lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(m0v)
               : "memory", "m0");
}
// As dma16_opaque, addressing global memory as a wave-uniform base plus this lane's unsigned
// 32-bit byte offset (the base lives in SGPRs, one VGPR per lane for the offset).
__device__ __forceinline__ void dma16_opaque_so(const void *sbase, uint32_t voff,
                                                uint32_t lds_base) {
  // readfirstlane works on int: each half goes back to uint32_t before widening, so the low
  // half is zero-extended (sign-extending it would corrupt the high half of the address)
  const uint64_t bp = (uint64_t)(uintptr_t)sbase;
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bp >> 32));
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bp);
  const uint64_t sb = ((uint64_t)bhi << 32) | (uint64_t)blo;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(m0v)
               : "memory", "m0");
}
// As dma16_opaque_so with 4 bytes per lane (lane i writes [lds_base + 4 i, +4)).
__device__ __forceinline__ void dma4_opaque_so(const void *sbase, uint32_t voff,
                                               uint32_t lds_base) {
  const uint64_t bp = (uint64_t)(uintptr_t)sbase;
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bp >> 32));
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bp);
  const uint64_t sb = ((uint64_t)bhi << 32) | (uint64_t)blo;
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(m0v)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// A pointer to LDS from a 32-bit LDS address (the inverse of lds_addr); the compiler infers
// the LDS address space from the cast, so accesses through it are LDS instructions.
template <typename U>
__device__ __forceinline__ U *lds_ptr(uint32_t addr) {
  return (U *)(__attribute__((address_space(3))) void *)(uintptr_t)addr;
}
// The same LDS address, opaque to the compiler: constant offsets from it then fold into the
// offset fields of the LDS instructions that use it. (From a loop-invariant address the
// compiler would form every base + offset ahead of the loop and hold each in a VGPR.)
__device__ __forceinline__ uint32_t lds_opaque(uint32_t addr) {
  asm volatile("" : "+v"(addr));
  return addr;
}

// ---------------------------------------------------------------- launch geometry
// Workgroup i runs on XCD (i mod 8). Map hardware ids so that logical ids
// [k*per, (k+1)*per) all run on XCD k in dispatch order: neighbouring tiles that
// share operands then share one L2.
__device__ __forceinline__ int xcd_remap(int i, int G) {
  const int per = G >> 3;
  const int full = per << 3;
  if (i >= full) return i;
  return (i & 7) * per + (i >> 3);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mm
