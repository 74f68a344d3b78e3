// The mixer's two dense contractions on bf16 MFMA (fp32 accumulate), and a plain fp32 path.
//
//   x_proj:  xdbl[T, R+2N] = u[T, D] . W_x[R+2N, D]^T           (fp32 out)
//   dt_proj: dt[T, D]      = softplus(dt_low[T, R] . W_dt[D, R]^T + b)   (fp32)
//
// Jamba analysis page, "The Mamba Layer", "The selective mechanism": B, C and Delta are
// functions of the token through small learned linear layers. Both products are "NT":
// every operand row is contiguous along the contraction, so one loader serves both.
//
// Precision: in bf16 I/O mode the activation operand is passed as two bf16 planes,
// a = a_hi + a_lo (a_hi = bf16(a), a_lo = bf16(a - a_hi)), and both are multiplied by the
// (exactly bf16) weights into the same fp32 accumulators: the product then carries the
// activation to ~2^-17 relative instead of bf16's 2^-9, at twice the MFMA work.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, lane layout checked on gfx950): the weight
// tile is the MFMA's first operand and the token tile its second, so each lane ends with
// 4 consecutive output columns of one token row -> 16-byte stores.
// A 256-thread workgroup computes a BM x BN tile as 2 x 2 waves; K advances in steps of 64
// through padded LDS tiles with the next step's global loads issued before the MFMAs.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kBK = 64;
constexpr int kPad = 8;              // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kPad;  // 72 elements = 144 bytes

struct EpiXproj {
  float *out;
  int ldo;
  __device__ __forceinline__ void operator()(int m, int n, const f32x4 &v) const {
    *(float4 *)(out + (int64_t)m * ldo + n) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

struct EpiDtprojF32 {
  float *out;
  const float *bias;
  int ldo;
  __device__ __forceinline__ void operator()(int m, int n, const f32x4 &v) const {
    const float4 b = *(const float4 *)(bias + n);
    *(float4 *)(out + (int64_t)m * ldo + n) =
        make_float4(softplus_f(v[0] + b.x), softplus_f(v[1] + b.y), softplus_f(v[2] + b.z),
                    softplus_f(v[3] + b.w));
  }
};

// C[M, N] = (A + A_lo)[M, K] . W[N, K]^T ; K % 64 == 0, N % 4 == 0; M, N otherwise arbitrary.
template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_nt_bf16_kernel(const bf16_t *__restrict__ A,
                                                           const bf16_t *__restrict__ A_lo,
                                                           const bf16_t *__restrict__ W, int M,
                                                           int N, int K, Epi epi) {
  constexpr int WM = BM / 2, WN = BN / 2;      // per-wave tile
  constexpr int MB = WM / 16, NB = WN / 16;    // 16x16 MFMA blocks per wave
  constexpr int A_CHUNKS = BM * kBK / 8;       // 16-byte chunks per tile
  constexpr int W_CHUNKS = BN * kBK / 8;
  constexpr int A_PER = (A_CHUNKS + 255) / 256;
  constexpr int W_PER = (W_CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t Als[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t Ws[BN * kLdsRow];

  const int ntn = (N + BN - 1) / BN;
  const int ntm = (M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, ntn * ntm);
  const int m0 = (lid / ntn) * BM;
  const int n0 = (lid % ntn) * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  uint4 ra[A_PER], ral[A_PER], rw[W_PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * 256;
      uint4 v = make_uint4(0, 0, 0, 0), vl = v;
      if (c < A_CHUNKS) {
        const int r = c >> 3, kc = (c & 7) * 8;
        if (m0 + r < M) {
          const int64_t off = (int64_t)(m0 + r) * K + k0 + kc;
          v = *(const uint4 *)(A + off);
          vl = *(const uint4 *)(A_lo + off);
        }
      }
      ra[i] = v;
      ral[i] = vl;
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
      const int c = tid + i * 256;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < W_CHUNKS) {
        const int r = c >> 3, kc = (c & 7) * 8;
        if (n0 + r < N) v = *(const uint4 *)(W + (int64_t)(n0 + r) * K + k0 + kc);
      }
      rw[i] = v;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * 256;
      if (c < A_CHUNKS) {
        *(uint4 *)(As + (c >> 3) * kLdsRow + (c & 7) * 8) = ra[i];
        *(uint4 *)(Als + (c >> 3) * kLdsRow + (c & 7) * 8) = ral[i];
      }
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
      const int c = tid + i * 256;
      if (c < W_CHUNKS) *(uint4 *)(Ws + (c >> 3) * kLdsRow + (c & 7) * 8) = rw[i];
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    stash();
    __syncthreads();
    if (k0 + kBK < K) load(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      const int koff = kk + (lane >> 4) * 8;
      bf16x8 fw[NB], fa[MB], fal[MB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fw[j] = __builtin_bit_cast(
            bf16x8, *(const uint4 *)(Ws + (wn * WN + j * 16 + (lane & 15)) * kLdsRow + koff));
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int ro = (wm * WM + i * 16 + (lane & 15)) * kLdsRow + koff;
        fa[i] = __builtin_bit_cast(bf16x8, *(const uint4 *)(As + ro));
        fal[i] = __builtin_bit_cast(bf16x8, *(const uint4 *)(Als + ro));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fal[i], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fa[i], acc[i][j], 0, 0, 0);
        }
    }
  }

  // acc[i][j] lane l: rows (weights) 4*(l/16)+r, column (token) l%16
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * WM + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + wn * WN + j * 16 + (lane >> 4) * 4;
      if (n < N) epi(m, n, acc[i][j]);
    }
  }
}

// fp32 path: one thread per output element, plain dot products (fp32 I/O mode).
// mode 0: out = acc (xdbl); mode 1: out = softplus(acc + bias[n]) (dt).
__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(const float *__restrict__ A,
                                                          const float *__restrict__ W, int M,
                                                          int N, int K, int mode,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)M * N) return;
  const int n = (int)(gid % N);
  const int64_t m = gid / N;
  const float *a = A + m * K;
  const float *w = W + (int64_t)n * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a[k], w[k], acc);
  out[gid] = mode == 0 ? acc : softplus_f(acc + bias[n]);
}

hipError_t f32_launch(const float *A, const float *W, int M, int N, int K, int mode,
                      const float *bias, float *out, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  hipLaunchKernelGGL(gemm_nt_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, A,
                     W, M, N, K, mode, bias, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_xproj(mm_dtype dt, const void *u, const void *u_lo, const void *w, float *xdbl,
                        int T, int D, int Nx, hipStream_t s) {
  if (dt == MM_F32) return f32_launch((const float *)u, (const float *)w, T, Nx, D, 0, nullptr, xdbl, s);
  constexpr int BM = 128, BN = 96;
  const int tiles = ((T + BM - 1) / BM) * ((Nx + BN - 1) / BN);
  EpiXproj e{xdbl, Nx};
  hipLaunchKernelGGL((gemm_nt_bf16_kernel<BM, BN, EpiXproj>), dim3(tiles), dim3(256), 0, s,
                     (const bf16_t *)u, (const bf16_t *)u_lo, (const bf16_t *)w, T, Nx, D, e);
  return hipGetLastError();
}

hipError_t launch_dtproj(mm_dtype dt, const void *dtlow, const void *dtlow_lo, const void *w,
                         const float *bias, void *dtout, int T, int D, int R, hipStream_t s) {
  if (dt == MM_F32)
    return f32_launch((const float *)dtlow, (const float *)w, T, D, R, 1, bias, (float *)dtout, s);
  constexpr int BM = 128, BN = 128;
  const int tiles = ((T + BM - 1) / BM) * ((D + BN - 1) / BN);
  EpiDtprojF32 e{(float *)dtout, bias, D};
  hipLaunchKernelGGL((gemm_nt_bf16_kernel<BM, BN, EpiDtprojF32>), dim3(tiles), dim3(256), 0, s,
                     (const bf16_t *)dtlow, (const bf16_t *)dtlow_lo, (const bf16_t *)w, T, D, R, e);
  return hipGetLastError();
}

}  // namespace mm
