// Selective scan + D feed-through + SiLU(z) gate + final SSM state.
//
// Jamba analysis page, "The Mamba Layer": every channel i runs its own scalar SSM with a
// diagonal A[i, :] over N states ("From scalar SSM to vector processing"); ZOH gives
// Abar = exp(dt A) (ZOH equation); the discrete recurrence h_t = Abar h_{t-1} + Bbar u_t,
// y_t = C_t h_t (recurrence equation); the continuous model's D u feed-through (continuous
// SSM equation). Bbar = dt B by default, or the page's ZOH form expm1(dt A)/A B with
// MM_FLAG_ZOH_B. Gate: y <- y * SiLU(z) (Mamba-1 block).
//
// The SSM input u = SiLU(conv1d(x) + b) is recomputed here in fp32 from x (4 taps per
// token, a sliding window in registers) instead of being read back rounded, so the scan
// sees u at full precision while reading no more bytes (x instead of u).
//
// Sequential kernel: one lane per (sequence, channel), all N = 16 states in VGPRs, B_t / C_t
// wave-uniform. Exactly one exp per (token, channel, state).
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

constexpr int kN = 16;

template <typename T> struct Delta;       // storage type of dt for each I/O dtype
template <> struct Delta<float> {
  typedef float type;
  static __device__ __forceinline__ float ld(const float *p) { return *p; }
};
template <> struct Delta<bf16_t> {
  typedef _Float16 type;
  static __device__ __forceinline__ float ld(const _Float16 *p) { return (float)*p; }
};

template <typename T, bool ZOH, int K>
__global__ __launch_bounds__(64) void scan_seq_kernel(ScanArgs a) {
  typedef typename Delta<T>::type DT;
  const int64_t gi = (int64_t)blockIdx.x * 64 + threadIdx.x;  // b * D + i
  const int i = (int)(gi % a.D);
  const int b = (int)(gi / a.D);
  float Av[kN], A2[kN], h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    Av[n] = a.A[(int64_t)i * kN + n];
    A2[n] = Av[n] * kLog2e;
    h[n] = (a.state_valid && a.state) ? a.state[gi * kN + n] : 0.0f;
  }
  const float Dv = a.Dskip[i];
  float w[K], win[K - 1];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = io<T>::cvt(((const T *)a.conv_w)[(int64_t)i * K + k]);
  const float cb = a.conv_b ? io<T>::cvt(((const T *)a.conv_b)[i]) : 0.0f;
#pragma unroll
  for (int j = 0; j < K - 1; ++j)
    win[j] = (a.conv_valid && a.conv_state)
                 ? io<T>::cvt(((const T *)a.conv_state)[gi * (K - 1) + j]) : 0.0f;

  const int64_t row = 2LL * a.D;
  const T *xp = (const T *)a.xz + (int64_t)b * a.L * row + i;
  const T *zp = xp + a.D;
  const DT *dp = (const DT *)a.delta + (int64_t)b * a.L * a.D + i;
  T *yp = (T *)a.y + (int64_t)b * a.L * a.D + i;
  const float *bcp = a.bc + (int64_t)b * a.L * 2 * kN;
  for (int t = 0; t < a.L; ++t) {
    const float x = io<T>::ld(xp + (int64_t)t * row);
    float acc = cb;
#pragma unroll
    for (int j = 0; j < K - 1; ++j) acc = __builtin_fmaf(w[j], win[j], acc);
    acc = __builtin_fmaf(w[K - 1], x, acc);
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
    win[K - 2] = x;
    const float u = silu_f(acc);
    const float dt = Delta<T>::ld(dp + (int64_t)t * a.D);
    const float z = io<T>::ld(zp + (int64_t)t * row);
    const float *Bt = bcp + (int64_t)t * 2 * kN;
    const float *Ct = Bt + kN;
    float y = 0.f;
    if (ZOH) {
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        const float em1 = expm1f(dt * Av[n]);
        const float dA = em1 + 1.0f;
        h[n] = __builtin_fmaf(dA, h[n], em1 / Av[n] * Bt[n] * u);
        y = __builtin_fmaf(Ct[n], h[n], y);
      }
    } else {
      const float dtu = dt * u;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        const float dA = exp2_hw(dt * A2[n]);
        h[n] = __builtin_fmaf(dA, h[n], dtu * Bt[n]);
        y = __builtin_fmaf(Ct[n], h[n], y);
      }
    }
    y = __builtin_fmaf(Dv, u, y) * silu_f(z);
    io<T>::st(yp + (int64_t)t * a.D, y);
  }
  if (a.state) {
#pragma unroll
    for (int n = 0; n < kN; ++n) a.state[gi * kN + n] = h[n];
  }
}

template <typename T, int K>
hipError_t dispatch_k(const ScanArgs &a, hipStream_t s) {
  const unsigned blocks = (unsigned)(((int64_t)a.B * a.D) / 64);
  if (a.zoh)
    hipLaunchKernelGGL((scan_seq_kernel<T, true, K>), dim3(blocks), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((scan_seq_kernel<T, false, K>), dim3(blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const ScanArgs &a, hipStream_t s) {
  switch (a.K) {
    case 2: return dispatch_k<T, 2>(a, s);
    case 3: return dispatch_k<T, 3>(a, s);
    case 4: return dispatch_k<T, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan(mm_dtype dt, const ScanArgs &a, hipStream_t s) {
  if (a.N != kN) return hipErrorInvalidValue;
  return dt == MM_BF16 ? dispatch<bf16_t>(a, s) : dispatch<float>(a, s);
}

}  // namespace mm
