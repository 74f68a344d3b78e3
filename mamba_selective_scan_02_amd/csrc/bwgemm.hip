// Split-precision bf16 products of the backward (bf16 I/O) and the operand planes they read.
//
// The backward's contractions (Jamba analysis page, "The Mamba Layer" and "The selective
// mechanism": x_proj and dt_proj are learned linear layers; their input and weight gradients
// are the transposed products) keep fp32 operands. Each is passed as two bf16 planes,
// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), which carries v to ~2^-17 relative. A
// product of two such operands is the sum of hi.hi + hi.lo + lo.hi (the dropped lo.lo term is
// below 2^-16 of each product); a product with a weight that is exactly bf16 is w.hi + w.lo.
// All terms go into one fp32 accumulator, on bf16 MFMA.
//
// gemm_sp_kernel   C[M, N] (+)= sum over segments s of A_s[M, K] . B_s[N, K]^T (rows of both
//                  operands contiguous along K, K % 64 == 0), fp32 out. 256 x 256 workgroup
//                  tiles of 8 waves (128 x 64 each, 32 16x16x32 accumulators); K advances in
//                  64-wide chunks through two 64 KB LDS stages filled by direct-to-LDS loads of
//                  whole 128-byte row segments (16-byte slot s of row r at s ^ ((r >> 1) & 7),
//                  so fragment reads are bank-conflict free), the next k-step's fragments read
//                  during the current MFMAs. The segments are walked one after another as one
//                  longer K loop. Rows past M or N read the last row and are not stored. A long
//                  K may be split over workgroups (blockIdx.y), each writing its own partial
//                  tile; sp_sum_kernel adds the partials in split order (deterministic).
// split_kernel     fp32 [rows, cols] -> hi / lo planes [rows, ldd], zero columns past cols.
// tsplit_kernel    fp32 [rows, cols] -> transposed hi / lo planes [cols, ldd], zero columns past
//                  rows (64 x 64 tiles through LDS), so that a product over the token axis
//                  reads both operands along their rows.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kT = 256;       // workgroup tile (M and N)
constexpr int kKc = 64;       // K chunk: one 128-byte segment of each operand row
constexpr int kGroupM = 4;    // tile order: groups of 4 row tiles sweep the column tiles

__global__ __launch_bounds__(512) void gemm_sp_kernel(SpGemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t a_s[2][kT][kKc];
  __shared__ __attribute__((aligned(16))) bf16_t b_s[2][kT][kKc];

  // the arguments as scalars: the lambdas below capture these, never the argument block itself
  // (which would then be copied to private memory)
  const int M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;
  const bf16_t *A0 = g.A[0], *A1 = g.A[1], *A2 = g.A[2];
  const bf16_t *B0 = g.B[0], *B1 = g.B[1], *B2 = g.B[2];
  // segment bases as integers, selected per chunk with masks
  const uint64_t uA0 = (uint64_t)A0, uA1 = (uint64_t)A1, uA2 = (uint64_t)A2;
  const uint64_t uB0 = (uint64_t)B0, uB1 = (uint64_t)B1, uB2 = (uint64_t)B2;
  const int nbn = (N + kT - 1) / kT, nbm = (M + kT - 1) / kT;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = gid / (kGroupM * nbn), gw = gid % (kGroupM * nbn);
  const int gm0 = grp * kGroupM, gsz = min(nbm - gm0, kGroupM);
  const int m0 = (gm0 + gw % gsz) * kT, n0 = (gw / gsz) * kT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;           // wave tile: rows 128 wm.., cols 64 wn..
  const int tl = lane & 15, gq = lane >> 4;

  // this workgroup's share [c0, c1) of the K / 64 chunks (the same range in every segment)
  const int nkt = g.K / kKc, z = blockIdx.y;
  const int c0 = (int)((int64_t)nkt * z / g.split);
  const int c1 = (int)((int64_t)nkt * (z + 1) / g.split);
  const int nk = c1 - c0, nc = nk * g.nseg;

  // Load q of wave wv covers rows 8 f .. 8 f + 7 of A (q < 4) or B (q >= 4), f = wv + 8 (q & 3):
  // lane l takes row 8 f + l / 8, physical slot l % 8, i.e. logical slot (l % 8) ^ sw(row).
  uint32_t voff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int f = wv + 8 * (q & 3);
    const int row = 8 * f + (lane >> 3);
    const int slot = (lane & 7) ^ ((row >> 1) & 7);
    const int grow = q < 4 ? min(m0 + row, M - 1) - m0 : min(n0 + row, N - 1) - n0;
    const int ld = q < 4 ? lda : ldb;
    voff[q] = (uint32_t)(((int64_t)grow * ld + slot * 8) * 2);
  }
  auto issue = [=](int kc) {
    const int sg = kc / nk, kk = c0 + kc % nk;
    const uint64_t k0 = 0ull - (uint64_t)(sg == 0), k1 = 0ull - (uint64_t)(sg == 1),
                   k2 = 0ull - (uint64_t)(sg == 2);
    const bf16_t *at = (const bf16_t *)((uA0 & k0) | (uA1 & k1) | (uA2 & k2)) +
                       (int64_t)m0 * lda + kk * kKc;
    const bf16_t *bt = (const bf16_t *)((uB0 & k0) | (uB1 & k1) | (uB2 & k2)) +
                       (int64_t)n0 * ldb + kk * kKc;
    const int st = kc & 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int f = wv + 8 * (q & 3);
      if (q < 4)
        dma16_opaque_so(at, voff[q], lds_addr(&a_s[st][8 * f][0]));
      else
        dma16_opaque_so(bt, voff[q], lds_addr(&b_s[st][8 * f][0]));
    }
  };
  const int sw = (tl >> 1) & 7;    // rows 16 b + tl all swizzle by (tl >> 1) & 7
  auto read_frags = [&](int st, int ks, bf16x8 (&fa)[8], bf16x8 (&fb)[4]) {
    const int col = ((4 * ks + gq) ^ sw) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = __builtin_bit_cast(bf16x8, *(const uint4 *)&b_s[st][wn * 64 + j * 16 + tl][col]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[i] = __builtin_bit_cast(bf16x8, *(const uint4 *)&a_s[st][wm * 128 + i * 16 + tl][col]);
  };

  f32x4 acc[4][8];   // [col block j][row block i]: C^T tile, see the epilogue
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const bf16x8 (&fa)[8], const bf16x8 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
  };

  // Pipeline: chunk kc + 1 is in flight to the other stage while chunk kc is multiplied; the
  // barrier between a chunk's two k-steps frees its stage for chunk kc + 2.
  if (nc > 0) {
    bf16x8 ca[8], cb[4], na[8], nb[4];
    issue(0);
    if (nc > 1) {
      issue(1);
      wait_vmem_le<8>();   // chunk 0 has landed (chunk 1's 8 loads may be in flight)
    } else {
      wait_vmem_all();
    }
    lds_barrier();
    read_frags(0, 0, ca, cb);
    for (int kc = 0; kc < nc; ++kc) {
      const int st = kc & 1;
      read_frags(st, 1, na, nb);
      mma(ca, cb);
      if (kc + 1 < nc) wait_vmem_all();   // chunk kc + 1 (the only loads in flight) has landed
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS reads are complete
      lds_barrier();       // every wave's reads of stage st are done; chunk kc + 1 is visible
      if (kc + 2 < nc) issue(kc + 2);
      if (kc + 1 < nc) read_frags(st ^ 1, 0, ca, cb);
      mma(na, nb);
    }
  }

  // epilogue: acc[j][i][r] = C[m0 + 128 wm + 16 i + tl][n0 + 64 wn + 16 j + 4 gq + r]
  float *out = g.C;
  int64_t ldo = g.ldc;
  bool add = g.accumulate != 0;
  if (g.split > 1) {
    out = g.part + (int64_t)z * g.M * g.N;
    ldo = g.N;
    add = false;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + wm * 128 + i * 16 + tl;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + gq * 4;
      if (n >= g.N) continue;
      float4 *o = (float4 *)(out + (int64_t)m * ldo + n);
      float4 v = make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
      if (add) {
        const float4 c = *o;
        v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
      }
      *o = v;
    }
  }
}

// C[m, n..n+3] (+)= sum over z of part[z][m][n..n+3], z in order
__global__ __launch_bounds__(256) void sp_sum_kernel(SpGemmArgs g) {
  const int nq = g.N / 4;
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= (int64_t)g.M * nq) return;
  const int64_t m = e / nq;
  const int n = (int)(e % nq) * 4;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z = 0; z < g.split; ++z) {
    const float4 p = *(const float4 *)(g.part + ((int64_t)z * g.M + m) * g.N + n);
    v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
  }
  float4 *o = (float4 *)(g.C + m * g.ldc + n);
  if (g.accumulate) {
    const float4 c = *o;
    v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
  }
  *o = v;
}

__device__ __forceinline__ void split2(float v, bf16_t &h, bf16_t &l) {
  h = f2bf(v);
  l = f2bf(v - bf2f(h));
}

// 4 consecutive columns per thread
__global__ __launch_bounds__(256) void split_kernel(const float *src, int64_t rows, int cols,
                                                    int64_t lds, bf16_t *hi, bf16_t *lo, int ldd) {
  const int nq = ldd / 4;
  const int64_t n = rows * nq;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / nq;
    const int c = (int)(e % nq) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < cols) v = *(const float4 *)(src + r * lds + c);
    bf16_t h[4], l[4];
    split2(v.x, h[0], l[0]);
    split2(v.y, h[1], l[1]);
    split2(v.z, h[2], l[2]);
    split2(v.w, h[3], l[3]);
    const int64_t o = r * ldd + c;
    *(uint2 *)(hi + o) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                    (uint32_t)h[2] | ((uint32_t)h[3] << 16));
    if (lo)
      *(uint2 *)(lo + o) = make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16),
                                      (uint32_t)l[2] | ((uint32_t)l[3] << 16));
  }
}

// dst[c][r] = src[r][c] for c < cols, r < ldd (zero for r >= rows); blockIdx.x: 64-row tile of
// src (64 columns of dst), blockIdx.y: 64-column tile of src
__global__ __launch_bounds__(256) void tsplit_kernel(const float *src, int rows, int cols,
                                                     int64_t lds, bf16_t *hi, bf16_t *lo,
                                                     int64_t ldd) {
  __shared__ float t_s[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = (tid >> 4) + 16 * q, cl = (tid & 15) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + rl < rows && c0 + cl < cols) v = *(const float4 *)(src + (int64_t)(r0 + rl) * lds + c0 + cl);
    t_s[rl][cl] = v.x;
    t_s[rl][cl + 1] = v.y;
    t_s[rl][cl + 2] = v.z;
    t_s[rl][cl + 3] = v.w;
  }
  __syncthreads();
  const int cl = tid >> 2, rl0 = (tid & 3) * 16;
  if (c0 + cl >= cols) return;
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bf16_t h0, l0, h1, l1;
    split2(t_s[rl0 + 2 * i][cl], h0, l0);
    split2(t_s[rl0 + 2 * i + 1][cl], h1, l1);
    h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  const int64_t o = (int64_t)(c0 + cl) * ldd + r0 + rl0;
  *(uint4 *)(hi + o) = make_uint4(h[0], h[1], h[2], h[3]);
  *(uint4 *)(hi + o + 8) = make_uint4(h[4], h[5], h[6], h[7]);
  if (lo) {
    *(uint4 *)(lo + o) = make_uint4(l[0], l[1], l[2], l[3]);
    *(uint4 *)(lo + o + 8) = make_uint4(l[4], l[5], l[6], l[7]);
  }
}

inline unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? b : 65536);
}

}  // namespace

int gemm_sp_split(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + kT - 1) / kT) * ((N + kT - 1) / kT);
  int split = 1;
  while (split < kSpMaxSplit && tiles * split < 1024 && (K / kKc) / (split * 2) >= 16) split *= 2;
  return split;
}

hipError_t launch_gemm_sp(const SpGemmArgs &g0, hipStream_t s) {
  if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
  SpGemmArgs g = g0;
  if (g.K <= 0 || g.K % kKc || g.N % 4 || g.ldc % 4 || g.nseg < 1 || g.nseg > 3 ||
      g.lda < g.K || g.ldb < g.K || g.lda % 8 || g.ldb % 8)
    return hipErrorInvalidValue;
  // lane offsets inside a 256-row tile are 32-bit byte offsets
  if ((int64_t)kT * (g.lda > g.ldb ? g.lda : g.ldb) * 2 >= (1ll << 32)) return hipErrorInvalidValue;
  g.split = g.part ? gemm_sp_split(g.M, g.N, g.K) : 1;
  const unsigned tiles = (unsigned)(((g.M + kT - 1) / kT) * ((g.N + kT - 1) / kT));
  hipLaunchKernelGGL(gemm_sp_kernel, dim3(tiles, (unsigned)g.split), dim3(512), 0, s, g);
  if (g.split > 1)
    hipLaunchKernelGGL(sp_sum_kernel, dim3((unsigned)(((int64_t)g.M * (g.N / 4) + 255) / 256)),
                       dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const float *src, int64_t rows, int cols, int64_t lds, bf16_t *hi,
                             bf16_t *lo, int ldd, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols % 4 || ldd % 4 || lds % 4 || ldd < cols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_kernel, dim3(grid_for(rows * (ldd / 4))), dim3(256), 0, s, src, rows,
                     cols, lds, hi, lo, ldd);
  return hipGetLastError();
}

hipError_t launch_tsplit_bf16(const float *src, int rows, int cols, int64_t lds, bf16_t *hi,
                              bf16_t *lo, int64_t ldd, hipStream_t s) {
  if (cols <= 0 || ldd <= 0) return hipSuccess;
  if (cols % 4 || lds % 4 || ldd % 64 || ldd < rows) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tsplit_kernel, dim3((unsigned)(ldd / 64), (unsigned)((cols + 63) / 64)),
                     dim3(256), 0, s, src, rows, cols, lds, hi, lo, ldd);
  return hipGetLastError();
}

}  // namespace mm
