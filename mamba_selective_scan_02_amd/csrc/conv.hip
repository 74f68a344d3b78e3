// Causal depthwise conv1d + bias + SiLU over the x half of xz, and the conv-state update.
//
// Not written out on the pages (the standard Mamba-1 block that the Jamba page's
// "The Mamba Layer" section builds on): u[b,t,i] = SiLU(bias_i + sum_k w[i,k] xt[b,t-(K-1)+k,i]),
// tap K-1 on the current token, with xt before token 0 taken from the carried state
// (oldest first) or zeros.
//
// In bf16 I/O mode u is written as two bf16 planes, u_hi = bf16(u) and u_lo = bf16(u - u_hi),
// so that x_proj sees u to ~2^-17 relative (two MFMA passes) instead of bf16's 2^-9.
//
// Layout / roofline: HBM-bound streaming kernel (read x: 2 B, write u: 4 B per element
// in bf16). Each thread owns VEC consecutive channels (16-byte loads and stores, so a
// wave touches 1 KB of contiguous row per token) and a run of TT consecutive tokens,
// keeping the K-1 previous inputs in registers; the K-1 halo rows are re-read once per
// run (3/TT extra reads).
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

constexpr int kTT = 32;  // tokens per thread

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  typedef float4 raw;
  static __device__ __forceinline__ void unpack(const raw &r, float *v) {
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  static __device__ __forceinline__ raw pack(const float *v) { return make_float4(v[0], v[1], v[2], v[3]); }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  typedef uint4 raw;
  static __device__ __forceinline__ void unpack(const raw &r, float *v) {
    v[0] = lo_bf(r.x); v[1] = hi_bf(r.x); v[2] = lo_bf(r.y); v[3] = hi_bf(r.y);
    v[4] = lo_bf(r.z); v[5] = hi_bf(r.z); v[6] = lo_bf(r.w); v[7] = hi_bf(r.w);
  }
  static __device__ __forceinline__ raw pack(const float *v) {
    raw r;
    r.x = pack_bf2(v[0], v[1]); r.y = pack_bf2(v[2], v[3]);
    r.z = pack_bf2(v[4], v[5]); r.w = pack_bf2(v[6], v[7]);
    return r;
  }
};

template <typename T, int K>
__global__ __launch_bounds__(256) void conv_silu_kernel(ConvArgs a) {
  typedef Vec<T> V;
  constexpr int VN = V::N;
  const int groups = a.D / VN;
  const int runs = (a.L + kTT - 1) / kTT;
  const int64_t total = (int64_t)a.B * runs * groups;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int g = (int)(gid % groups);
  const int64_t rest = gid / groups;
  const int run = (int)(rest % runs);
  const int b = (int)(rest / runs);
  const int c0 = g * VN;
  const int t0 = run * kTT;
  const int t1 = min(a.L, t0 + kTT);

  const T *wp = (const T *)a.w;
  float w[VN][K];
  float bias[VN];
#pragma unroll
  for (int v = 0; v < VN; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[v][k] = io<T>::cvt(wp[(int64_t)(c0 + v) * K + k]);
    bias[v] = a.bias ? io<T>::cvt(((const T *)a.bias)[c0 + v]) : 0.0f;
  }

  const int64_t row = 2LL * a.D;  // xz row stride in elements
  const T *xb = (const T *)a.xz + (int64_t)b * a.L * row + c0;
  float win[K > 1 ? K - 1 : 1][VN];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int tau = t0 - (K - 1) + j;
    if (tau >= 0) {
      V::unpack(*(const typename V::raw *)(xb + (int64_t)tau * row), win[j]);
    } else if (a.state_valid && a.state) {
      const T *sp = (const T *)a.state + ((int64_t)b * a.D + c0) * (K - 1) + (K - 1 + tau);
#pragma unroll
      for (int v = 0; v < VN; ++v) win[j][v] = io<T>::cvt(sp[(int64_t)v * (K - 1)]);
    } else {
#pragma unroll
      for (int v = 0; v < VN; ++v) win[j][v] = 0.0f;
    }
  }

  T *ub = (T *)a.u + (int64_t)b * a.L * a.D + c0;
  T *ulb = (T *)a.u_lo + (int64_t)b * a.L * a.D + c0;  // bf16 only
  for (int t = t0; t < t1; ++t) {
    float cur[VN], out[VN];
    V::unpack(*(const typename V::raw *)(xb + (int64_t)t * row), cur);
#pragma unroll
    for (int v = 0; v < VN; ++v) {
      float acc = bias[v];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc = __builtin_fmaf(w[v][j], win[j][v], acc);
      acc = __builtin_fmaf(w[v][K - 1], cur[v], acc);
      out[v] = silu_f(acc);
    }
    *(typename V::raw *)(ub + (int64_t)t * a.D) = V::pack(out);
    if (sizeof(T) == 2) {
      // low part: u - bf16(u), exact in fp32, then rounded to bf16 (u = hi + lo to ~2^-17)
      float lo[VN];
#pragma unroll
      for (int v = 0; v < VN; ++v) lo[v] = out[v] - bf2f(f2bf(out[v]));
      *(typename V::raw *)(ulb + (int64_t)t * a.D) = V::pack(lo);
    }
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
      for (int v = 0; v < VN; ++v) win[j][v] = win[j + 1][v];
    if (K > 1) {
#pragma unroll
      for (int v = 0; v < VN; ++v) win[K - 2][v] = cur[v];
    }
  }
}

// One thread per (b, i): new_state[j] = xt[L + j] where xt = concat(old_state, x).
template <typename T, int K>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a, T *state) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.B * a.D) return;
  const int i = (int)(gid % a.D);
  const int b = (int)(gid / a.D);
  T *sp = state + gid * (K - 1);
  float old[K - 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) old[j] = a.state_valid ? io<T>::cvt(sp[j]) : 0.0f;
  const T *xb = (const T *)a.xz + (int64_t)b * a.L * 2 * a.D + i;
  float nw[K - 1];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int m = a.L + j;  // index into xt
    nw[j] = (m < K - 1) ? old[m] : io<T>::cvt(xb[(int64_t)(m - (K - 1)) * 2 * a.D]);
  }
#pragma unroll
  for (int j = 0; j < K - 1; ++j) io<T>::st(sp + j, nw[j]);
}

template <typename T, int K>
hipError_t conv_dispatch(const ConvArgs &a, hipStream_t s) {
  const int groups = a.D / Vec<T>::N;
  const int runs = (a.L + kTT - 1) / kTT;
  const int64_t total = (int64_t)a.B * runs * groups;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL((conv_silu_kernel<T, K>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t state_dispatch(const ConvArgs &a, void *state, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.D;
  hipLaunchKernelGGL((conv_state_kernel<T, K>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     s, a, (T *)state);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_silu(mm_dtype dt, const ConvArgs &a, hipStream_t s) {
  if (dt == MM_BF16) {
    switch (a.K) {
      case 2: return conv_dispatch<bf16_t, 2>(a, s);
      case 3: return conv_dispatch<bf16_t, 3>(a, s);
      case 4: return conv_dispatch<bf16_t, 4>(a, s);
    }
  } else {
    switch (a.K) {
      case 2: return conv_dispatch<float, 2>(a, s);
      case 3: return conv_dispatch<float, 3>(a, s);
      case 4: return conv_dispatch<float, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_state_update(mm_dtype dt, const ConvArgs &a, void *state_out, hipStream_t s) {
  if (dt == MM_BF16) {
    switch (a.K) {
      case 2: return state_dispatch<bf16_t, 2>(a, state_out, s);
      case 3: return state_dispatch<bf16_t, 3>(a, state_out, s);
      case 4: return state_dispatch<bf16_t, 4>(a, state_out, s);
    }
  } else {
    switch (a.K) {
      case 2: return state_dispatch<float, 2>(a, state_out, s);
      case 3: return state_dispatch<float, 3>(a, state_out, s);
      case 4: return state_dispatch<float, 4>(a, state_out, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mm
