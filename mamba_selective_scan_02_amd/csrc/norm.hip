// RMSNorm of the three x_proj slices of every token (dt_low over R, B over N, C over N).
//
// Jamba analysis page, "RMSNorm definition and placement" (RMSNorm equation:
// v / sqrt(mean(v^2) + eps) * gamma) applied to the mixer's internal activations per
// "Stabilization: RMSNorm in Mamba layers". One wave per token; each slice's sum of
// squares is a wave reduction. Traffic is ~2 KB per token (read xdbl fp32, write dt_low
// in the I/O dtype and B|C in fp32), negligible next to the scan's ~64 KB per token.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void norm_kernel(const float *__restrict__ xdbl,
                                                   T *__restrict__ dtlow, T *__restrict__ dtlow_lo,
                                                   float *__restrict__ bc,
                                                   const float *__restrict__ g_dt,
                                                   const float *__restrict__ g_B,
                                                   const float *__restrict__ g_C, int T_, int R,
                                                   int N, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int W = R + 2 * N;
  const float *row = xdbl + t * W;
  float ss = 0.f;
  for (int r = lane; r < R; r += 64) {
    const float v = row[r];
    ss = __builtin_fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  const float inv_dt = 1.0f / sqrtf(ss / (float)R + eps);
  for (int r = lane; r < R; r += 64) {
    const float v = row[r] * inv_dt * g_dt[r];
    io<T>::st(dtlow + t * R + r, v);
    // bf16 mode: the low part carries v - bf16(v) for dt_proj's second MFMA pass
    if (sizeof(T) == 2) io<T>::st(dtlow_lo + t * R + r, v - bf2f(f2bf(v)));
  }
  // B = row[R, R+N), C = row[R+N, R+2N); lane j takes elements j, j + 64, ... (N <= 64)
  float sb = 0.f, sc = 0.f;
  for (int j = lane; j < N; j += 64) {
    const float vb = row[R + j], vc = row[R + N + j];
    sb = __builtin_fmaf(vb, vb, sb);
    sc = __builtin_fmaf(vc, vc, sc);
  }
  sb = wave_sum(sb);
  sc = wave_sum(sc);
  const float ib = 1.0f / sqrtf(sb / (float)N + eps), ic = 1.0f / sqrtf(sc / (float)N + eps);
  for (int j = lane; j < N; j += 64) {
    bc[t * 2 * N + j] = row[R + j] * ib * g_B[j];
    bc[t * 2 * N + N + j] = row[R + N + j] * ic * g_C[j];
  }
}

}  // namespace

hipError_t launch_norm(mm_dtype dt, const float *xdbl, void *dtlow, void *dtlow_lo, float *bc,
                       const float *g_dt, const float *g_B, const float *g_C, int T, int R, int N,
                       float eps, hipStream_t s) {
  const unsigned blocks = (unsigned)((T + 3) / 4);
  if (dt == MM_BF16)
    hipLaunchKernelGGL(norm_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, xdbl, (bf16_t *)dtlow,
                       (bf16_t *)dtlow_lo, bc, g_dt, g_B, g_C, T, R, N, eps);
  else
    hipLaunchKernelGGL(norm_kernel<float>, dim3(blocks), dim3(256), 0, s, xdbl, (float *)dtlow,
                       (float *)nullptr, bc, g_dt, g_B, g_C, T, R, N, eps);
  return hipGetLastError();
}

}  // namespace mm
