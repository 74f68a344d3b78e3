// Mamba layer around the mixer (bf16 I/O): pre-RMSNorm, in_proj, the mixer, out_proj with the
// residual added.
//
// Jamba analysis page, "The Mamba Layer": the input hidden state is projected linearly to the
// d_inner independent scalar SSMs and their concatenated outputs are projected back ("From
// scalar SSM to vector processing", steps 1 and 4); "RMSNorm definition and placement": RMSNorm
// at the input of every Mamba module (RMSNorm equation). The residual add around the module is
// the standard pre-norm block the architecture description implies.
//
//   out = x + W_out . mixer(W_in . RMSNorm(x))
//
// rmsnorm_rows_kernel   one wave per token: x / sqrt(mean(x^2) + eps) * g, bf16 out.
// gemm256_kernel        C[M, N] = A[M, K] . B[N, K]^T (+ R[M, N]), bf16 in, fp32 accumulate, bf16
//                       out, N % 256 == 0. 256 x 256 workgroup tiles, 8 waves (two per SIMD) of
//                       128 x 64 (32 independent 16x16x32 MFMA accumulators each). K advances in
//                       chunks of 64 through two LDS stages (64 KB each) filled by direct-to-LDS
//                       loads one chunk ahead; every load instruction brings 8 whole 128-byte
//                       rows, stored with the 16-byte slot s of row r at s ^ ((r >> 1) & 7) so
//                       that the MFMA fragment reads hit distinct banks. Fragments of the next
//                       k-step are read while the current one's MFMAs run; tiles are ordered in
//                       groups of 4 row tiles per column tile so that an XCD's tiles in flight
//                       share operands in its L2. The larger tile halves the operand bytes per
//                       flop of a 128 x 128 tile: at the MFMA rate a 128 x 128 tile needs more
//                       L2 -> LDS bandwidth than the chip delivers.
// gemm_nt_kernel        the same product for N % 128 == 0 (narrow layers): 128 x 128 tiles, 4
//                       waves of 64 x 64; operand tiles in LDS in MFMA fragment order (each
//                       16 x 32 fragment is 1 KB with lane i's 16 bytes at 16 i), 3 stages.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kBM = 128, kBN = 128, kBK = 64;   // workgroup tile and K chunk
constexpr int kStages = 3;
constexpr int kFragA = (kBM / 16) * (kBK / 32);  // 1 KB fragments per stage: 16
constexpr int kFragB = (kBN / 16) * (kBK / 32);  //                            16
constexpr int kLoadsPerWave = (kFragA + kFragB) / 4;   // 8

__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmArgs g) {
  // [stage][fragment][64 lanes x 8 bf16]; fragment f = row block (f >> 1), k-step (f & 1)
  __shared__ __attribute__((aligned(16))) bf16_t a_s[kStages][kFragA][512];
  __shared__ __attribute__((aligned(16))) bf16_t b_s[kStages][kFragB][512];

  const int nbn = g.N / kBN;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (gid / nbn) * kBM, n0 = (gid % nbn) * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;           // wave tile: rows 64 wm.., cols 64 wn..
  const int tl = lane & 15, gq = lane >> 4;
  const int nk = g.K / kBK;

  // Wave wv issues fragment loads wv, wv + 4, ... of the stage's 32 (A first, then B). Fragment
  // lane l: row 16 rb + l % 16, k = k0 + 32 ks + 8 (l / 16) .. +7. Rows past M read row M-1.
  auto issue = [&](int kc) {
    const int k0 = kc * kBK;
    const int st = kc % kStages;
#pragma unroll
    for (int q = 0; q < kLoadsPerWave; ++q) {
      const int f = wv + 4 * q;
      if (f < kFragA) {
        const int rb = f >> 1, ks = f & 1;
        const int r = min(m0 + rb * 16 + tl, g.M - 1);
        dma16_opaque(g.A + (int64_t)r * g.K + k0 + ks * 32 + gq * 8, lds_addr(&a_s[st][f][0]));
      } else {
        const int fb = f - kFragA;
        const int rb = fb >> 1, ks = fb & 1;
        const int r = n0 + rb * 16 + tl;
        dma16_opaque(g.B + (int64_t)r * g.K + k0 + ks * 32 + gq * 8, lds_addr(&b_s[st][fb][0]));
      }
    }
  };

  f32x4 acc[4][4];   // [col block j][row block i]: C^T tile, see the epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue(0);
  if (nk > 1) issue(1);
  for (int kc = 0; kc < nk; ++kc) {
    // chunk kc's loads have landed (only chunk kc+1's may still be in flight)
    if (kc + 1 < nk) wait_vmem_le<kLoadsPerWave>();
    else wait_vmem_all();
    lds_barrier();     // every wave's loads for kc are visible; stage (kc+2) % 3 is free
    if (kc + 2 < nk) issue(kc + 2);
    const int st = kc % kStages;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = __builtin_bit_cast(bf16x8, *(const uint4 *)&a_s[st][(wm * 4 + i) * 2 + ks][lane * 8]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = __builtin_bit_cast(bf16x8, *(const uint4 *)&b_s[st][(wn * 4 + j) * 2 + ks][lane * 8]);
      // D = B_frag . A_frag^T: lane (tl, gq) gets C[row 16 i + tl][cols 16 j + 4 gq .. +3]
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
    }
  }

  // epilogue: acc[j][i][r] = C[m0 + 64 wm + 16 i + tl][n0 + 64 wn + 16 j + 4 gq + r]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + i * 16 + tl;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + gq * 4;
      float v0 = acc[j][i][0], v1 = acc[j][i][1], v2 = acc[j][i][2], v3 = acc[j][i][3];
      if (g.R) {
        const uint2 rr = *(const uint2 *)(g.R + (int64_t)m * g.ldr + n);
        v0 += lo_bf(rr.x); v1 += hi_bf(rr.x); v2 += lo_bf(rr.y); v3 += hi_bf(rr.y);
      }
      uint2 o;
      o.x = pack_bf2(v0, v1);
      o.y = pack_bf2(v2, v3);
      *(uint2 *)(g.C + (int64_t)m * g.ldc + n) = o;
    }
  }
}

constexpr int kT2 = 256;        // gemm256 tile (M and N)
constexpr int kK2 = 64;         // K chunk: one 128-byte row segment per operand row

constexpr int kGroupM = 4;      // tile order: groups of 4 row tiles sweep the column tiles

__global__ __launch_bounds__(512) void gemm256_kernel(GemmArgs g) {
  // [stage][row][64 bf16]: row r holds its chunk's 8 slots of 16 bytes, slot s at s ^ sw(r)
  __shared__ __attribute__((aligned(16))) bf16_t a_s[2][kT2][kK2];
  __shared__ __attribute__((aligned(16))) bf16_t b_s[2][kT2][kK2];

  // Tile order: consecutive ids (which share an XCD and its L2) walk kGroupM row tiles for each
  // column tile, so the tiles in flight on one XCD share both A row blocks and B column blocks.
  const int nbn = g.N / kT2, nbm = (g.M + kT2 - 1) / kT2;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = gid / (kGroupM * nbn), gw = gid % (kGroupM * nbn);
  const int gm0 = grp * kGroupM, gsz = min(nbm - gm0, kGroupM);
  const int m0 = (gm0 + gw % gsz) * kT2, n0 = (gw / gsz) * kT2;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;           // wave tile: rows 128 wm.., cols 64 wn..
  const int tl = lane & 15, gq = lane >> 4;
  const int nk = g.K / kK2;
  const bf16_t *at = g.A + (int64_t)m0 * g.K;    // tile bases; lane offsets stay below 2^32
  const bf16_t *bt = g.B + (int64_t)n0 * g.K;

  // Load q of wave wv covers rows 8 f .. 8 f + 7 of A (q < 4) or B (q >= 4), f = wv + 8 (q & 3):
  // lane l takes row 8 f + l / 8, physical slot l % 8, i.e. logical slot (l % 8) ^ sw(row).
  // A rows past M read row M - 1 (their results are not stored).
  uint32_t voff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int f = wv + 8 * (q & 3);
    const int row = 8 * f + (lane >> 3);
    const int slot = (lane & 7) ^ ((row >> 1) & 7);
    const int grow = q < 4 ? min(m0 + row, g.M - 1) - m0 : row;
    voff[q] = (uint32_t)((grow * g.K + slot * 8) * 2);
  }
  auto issue = [&](int kc) {
    const int st = kc & 1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int f = wv + 8 * (q & 3);
      if (q < 4)
        dma16_opaque_so(at + kc * kK2, voff[q], lds_addr(&a_s[st][8 * f][0]));
      else
        dma16_opaque_so(bt + kc * kK2, voff[q], lds_addr(&b_s[st][8 * f][0]));
    }
  };
  // this wave's operand fragments of k-step ks (32 wide) of the chunk in stage st
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
  // D = B_frag . A_frag^T: lane (tl, gq) gets C[row 16 i + tl][cols 16 j + 4 gq .. +3]
  auto mma = [&](const bf16x8 (&fa)[8], const bf16x8 (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[j][i], 0, 0, 0);
  };

  // Pipeline: chunk kc + 1 is in flight to the other stage while chunk kc is multiplied, and
  // the fragments of the next k-step are read from LDS while the current one's MFMAs run. The
  // barrier sits between a chunk's two k-steps: by then every wave holds all of that chunk's
  // fragments, so its stage can take chunk kc + 2.
  bf16x8 ca[8], cb[4], na[8], nb[4];
  issue(0);
  if (nk > 1) {
    issue(1);
    wait_vmem_le<8>();   // chunk 0 has landed (chunk 1's 8 loads may be in flight)
  } else {
    wait_vmem_all();
  }
  lds_barrier();
  read_frags(0, 0, ca, cb);
  for (int kc = 0; kc < nk; ++kc) {
    const int st = kc & 1;
    read_frags(st, 1, na, nb);
    mma(ca, cb);
    if (kc + 1 < nk) wait_vmem_all();   // chunk kc + 1 (the only loads in flight) has landed
    // lgkmcnt(0) as a builtin, so the compiler knows the reads above are complete and does not
    // wait on the next reads before the MFMAs below; the barrier's own wait repeats it
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();       // every wave's reads of stage st are done; chunk kc + 1 is visible
    if (kc + 2 < nk) issue(kc + 2);
    if (kc + 1 < nk) read_frags(st ^ 1, 0, ca, cb);
    mma(na, nb);
  }

  // epilogue: acc[j][i][r] = C[m0 + 128 wm + 16 i + tl][n0 + 64 wn + 16 j + 4 gq + r]
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + wm * 128 + i * 16 + tl;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + gq * 4;
      float v0 = acc[j][i][0], v1 = acc[j][i][1], v2 = acc[j][i][2], v3 = acc[j][i][3];
      if (g.R) {
        const uint2 rr = *(const uint2 *)(g.R + (int64_t)m * g.ldr + n);
        v0 += lo_bf(rr.x); v1 += hi_bf(rr.x); v2 += lo_bf(rr.y); v3 += hi_bf(rr.y);
      }
      uint2 o;
      o.x = pack_bf2(v0, v1);
      o.y = pack_bf2(v2, v3);
      *(uint2 *)(g.C + (int64_t)m * g.ldc + n) = o;
    }
  }
}

// One wave per token: y = x / sqrt(mean(x^2) + eps) * gamma (bf16 in and out, fp32 math).
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const bf16_t *x, const float *gamma,
                                                           bf16_t *y, int T, int Dm, float eps) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const bf16_t *xr = x + (int64_t)t * Dm;
  float ss = 0.f;
  for (int c = lane * 8; c < Dm; c += 512) {
    const uint4 v = *(const uint4 *)(xr + c);
    const float f[8] = {lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y),
                        lo_bf(v.z), hi_bf(v.z), lo_bf(v.w), hi_bf(v.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)Dm + eps);
  bf16_t *yr = y + (int64_t)t * Dm;
  for (int c = lane * 8; c < Dm; c += 512) {
    const uint4 v = *(const uint4 *)(xr + c);
    const float4 g0 = *(const float4 *)(gamma + c), g1 = *(const float4 *)(gamma + c + 4);
    uint4 o;
    o.x = pack_bf2(lo_bf(v.x) * inv * g0.x, hi_bf(v.x) * inv * g0.y);
    o.y = pack_bf2(lo_bf(v.y) * inv * g0.z, hi_bf(v.y) * inv * g0.w);
    o.z = pack_bf2(lo_bf(v.z) * inv * g1.x, hi_bf(v.z) * inv * g1.y);
    o.w = pack_bf2(lo_bf(v.w) * inv * g1.z, hi_bf(v.w) * inv * g1.w);
    *(uint4 *)(yr + c) = o;
  }
}

}  // namespace

bool gemm_nt_supported(int M, int N, int K) {
  return M > 0 && N > 0 && K > 0 && N % kBN == 0 && K % kBK == 0;
}

hipError_t launch_gemm_nt(const GemmArgs &g, hipStream_t s, int tile) {
  // 256 x 256 tiles once they fill the chip; below that the 4x as many 128 x 128 tiles spread
  // the work over more CUs
  if (tile == 0)
    tile = (g.N % kT2 == 0 && (int64_t)((g.M + kT2 - 1) / kT2) * (g.N / kT2) >= 256) ? kT2 : kBN;
  if (tile == kT2 && g.N % kT2 == 0) {
    const int grid = ((g.M + kT2 - 1) / kT2) * (g.N / kT2);
    hipLaunchKernelGGL(gemm256_kernel, dim3((unsigned)grid), dim3(512), 0, s, g);
  } else {
    const int grid = ((g.M + kBM - 1) / kBM) * (g.N / kBN);
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)grid), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const bf16_t *x, const float *gamma, bf16_t *y, int T, int Dm,
                               float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, gamma,
                     y, T, Dm, eps);
  return hipGetLastError();
}

}  // namespace mm
