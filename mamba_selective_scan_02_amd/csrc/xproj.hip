// Fused conv1d + SiLU -> x_proj (split-precision bf16 MFMA) -> RMSNorm of dt_low, B, C.
//
// Jamba analysis page: "The selective mechanism" (B, C and Delta from small linear layers of
// the token) and "RMSNorm definition and placement" / "Stabilization: RMSNorm in Mamba layers"
// (RMSNorm on the mixer's internal activations). The conv1d + SiLU producing the projection's
// input is the standard Mamba-1 block the page builds on.
//
// Design (bf16 I/O, dt_rank = 16 * RB, d_state N = 8, 16 or 32):
//   * One workgroup = a tile of 128 consecutive tokens of one sequence and ALL R + 2N outputs
//     of those tokens, so every (token, channel) input u is formed once and the three RMSNorms
//     run in the epilogue (xdbl never goes to memory).
//   * The contraction over d_inner advances in chunks of 32 channels (one MFMA k-step) through
//     a producer / consumer pipeline with one workgroup barrier per chunk:
//       - producer waves 0..7 (lane = one token x 8 channels) form u = SiLU(conv1d(x) + b) of
//         chunk i in fp32 (the 4-tap conv as two packed bf16 dot products per channel), split
//         it as u = hi + lo (both bf16) and write both into LDS; they also issue the
//         direct-to-LDS loads of the x rows, conv taps and W_x rows of chunk i + 2;
//       - consumer waves 8..15 multiply chunk i - 1: wave 8 + c owns tokens 32 (c % 4) .. +31
//         and one half of the output rows, two MFMAs (u_lo, u_hi) per W fragment and token
//         block (each W fragment read from LDS feeds four), so the product carries u to
//         ~2^-17 relative.
//     Each SIMD runs two producer and two consumer waves (<= 128 VGPRs each), so the VALU
//     work of one role overlaps the MFMAs of the other.
//     W_x chunks are 4-deep buffered, x rows (128 B = two chunks per stage) 2-deep, u
//     2-deep. W_x and u are stored in MFMA fragment order (each 16 x 32 operand block is 1 KB
//     with lane i's 16 bytes at 16 i), so every fragment read is one contiguous,
//     bank-conflict-free 1 KB access; x rows have their 16-byte slots XOR-swizzled by row.
//   * Epilogue (consumers): lane (token, 4 consecutive outputs per 16-wide block) squares and
//     sums its dt_low / B / C values, the 4 lanes of a token reduce by lane shuffles, the two
//     halves' sums meet through LDS, and the normalised dt_low (as bf16 hi + lo for dt_proj)
//     and B|C (fp32) are written.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTok = 128;          // tokens per workgroup
constexpr int kKC = 32;            // channels per chunk (one MFMA k-step)
constexpr int kXR = 144;           // staged x rows: 3 before the tile + 128, padded to 16-row loads

// physical 16-byte slot of logical slot c (0..7) in a 128-byte x row r (conflict-free reads of
// one logical slot of consecutive rows)
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int RB, int K, int N>
__global__ __launch_bounds__(1024) void xproj_fused_kernel(XprojFusedArgs a) {
  static_assert(K == 4, "the staged conv taps are laid out as [channel][4]");
  static_assert(N == 8 || N == 16 || N == 32, "B | C fill whole 16-row blocks");
  constexpr int R = RB * 16;
  constexpr int NX = R + 2 * N;        // outputs: dt_low | B | C
  constexpr int NB = NX / 16;          // 16-row MFMA blocks
  constexpr int LW = NX / 16;          // 1 KB wave-loads per chunk: W_x rows
  constexpr int PW = (LW + 7) / 8;     // W_x loads per producer wave (padded)
  // x rows are staged 128 B wide (two chunks, 64 channels): every row is one whole 128-byte
  // line (rows are 2 d_inner apart in memory, so half lines would be evicted before the
  // second half is read). One x stage = kXR rows = kXR / 8 wave-loads, issued with the loads
  // of every even chunk.
  constexpr int LX = kXR / 8;
  constexpr int PXS = (LX + 7) / 8;    // x loads per producer wave per x stage (padded)
  constexpr int PODD = PW + 1;         // loads per producer wave issued for an odd chunk
  constexpr int PEVEN = PW + 1 + PXS;  //                                   an even chunk
  __shared__ __attribute__((aligned(16))) bf16_t w_s[4][NB][64 * 8];   // fragment order
  __shared__ __attribute__((aligned(16))) bf16_t x_s[2][kXR][2 * kKC];   // x stages
  __shared__ __attribute__((aligned(16))) bf16_t u_s[2][2][kTok / 16][64 * 8];  // [buf][hi, lo]
  __shared__ __attribute__((aligned(16))) bf16_t cw_s[3][kKC * 4];       // conv taps [ch][4]
  __shared__ __attribute__((aligned(16))) bf16_t cb_s[3][kKC];           // conv bias
  __shared__ __attribute__((aligned(16))) float ss_s[8][32][4];           // consumers' sums

  const int tiles_per_seq = (a.L + kTok - 1) / kTok;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = gid / tiles_per_seq;
  const int t0 = (gid % tiles_per_seq) * kTok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar role / load branches
  const bool producer = wv < 8;
  const int64_t row = 2LL * a.D;
  const bf16_t *xzb = a.xz + (int64_t)b * a.L * row;
  const int Lm1 = a.L - 1;
  const int nck = a.D / kKC;

  // Producer wave wv issues W_x loads wv, wv + 8, ... of chunk ck, load wv of the list
  // [taps | bias] (the other waves repeat the taps load, which rewrites the same bytes) and,
  // for an even chunk, x loads wv, wv + 8, ... of x stage ck / 2; indices past a list repeat
  // its load 0. So every producer wave issues PEVEN loads for an even chunk and PODD for an
  // odd one. Addresses are wave-uniform bases plus unsigned 32-bit lane offsets.
  const int xrow0 = max(t0 - 3, 0);                 // x rows are read relative to this token
  const bf16_t *xbase = xzb + (int64_t)xrow0 * row;
  const bf16_t *bsrc = a.conv_b ? a.conv_b : a.conv_w;  // without a bias: the taps, unused
  auto issue = [&](int ck) {
    const int c0 = ck * kKC;
    const int b3 = ck % 3, b4 = ck & 3;
#pragma unroll
    for (int q = 0; q < PW; ++q) {
      int ld = wv + 8 * q;                          // = 16-row block nb of W_x
      if (ld >= LW) ld = 0;
      // fragment lane l: row 16 nb + l % 16, channels c0 + 8 (l / 16) .. +7
      const int r = ld * 16 + (lane & 15);
      dma16_opaque_so(a.w, (uint32_t)(r * a.D + c0 + (lane >> 4) * 8) * 2u,
                      lds_addr(&w_s[b4][ld][0]));
    }
    if (wv == 1) {
      if (lane < 4)
        dma16_opaque_so(bsrc, (uint32_t)(c0 + lane * 8) * 2u, lds_addr(&cb_s[b3][0]));
    } else {
      if (lane < 16)
        dma16_opaque_so(a.conv_w, (uint32_t)(c0 * K + lane * 8) * 2u, lds_addr(&cw_s[b3][0]));
    }
    if ((ck & 1) == 0) {
      const int xb = (ck >> 1) & 1;
#pragma unroll
      for (int q = 0; q < PXS; ++q) {
        int li = wv + 8 * q;
        if (li >= LX) li = 0;
        const int r = li * 8 + (lane >> 3), ps = lane & 7;
        const int tt = min(max(t0 - 3 + r, 0), Lm1) - xrow0;   // row r <-> token t0 - 3 + r
        dma16_opaque_so(xbase, (uint32_t)(tt * (int)row + c0 + swz8(r, ps) * 8) * 2u,
                        lds_addr(&x_s[xb][li * 8][0]));
      }
    }
  };

  // ---- producer: u of chunk ck for token ptok and channel group pgrp (8 channels)
  const int pidx = wv * 64 + lane;              // producers: 0 .. 511
  const int ptok = pidx & (kTok - 1), pgrp = (pidx >> 7) & 3;
  auto produce = [&](int ck) {
    const int c0 = ck * kKC;
    const int b3 = ck % 3;
    const int xb = (ck >> 1) & 1, xs0 = (ck & 1) * 4;   // x stage buffer, logical slot base
    {
      const int grp = pgrp;
      uint32_t xr[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = ptok + j;                  // rows ptok .. ptok+3: tokens t-3 .. t
        const uint4 v = *(const uint4 *)&x_s[xb][r][swz8(r, xs0 + grp) * 8];
        xr[j][0] = v.x; xr[j][1] = v.y; xr[j][2] = v.z; xr[j][3] = v.w;
      }
      if (t0 == 0 && ptok < 3) {
        // rows before token 0: carried conv state (oldest first) or zeros
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int tt = ptok + j - 3;
          if (tt < 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              uint32_t w = 0;
              if (a.conv_valid && a.conv_state) {
                const int64_t s0 = ((int64_t)b * a.D + c0 + grp * 8 + 2 * k) * (K - 1) + (K - 1) + tt;
                w = (uint32_t)a.conv_state[s0] | ((uint32_t)a.conv_state[s0 + (K - 1)] << 16);
              }
              xr[j][k] = w;
            }
          }
        }
      }
      // conv = (x_{t-3}, x_{t-2}) . (w0, w1) + (x_{t-1}, x_t) . (w2, w3) + b: each pair of
      // window rows of one channel is gathered into one bf16x2 (v_perm) and multiplied with
      // the channel's packed taps (v_dot2, fp32 accumulate)
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cl = grp * 8 + e;
        const uint2 wr = *(const uint2 *)&cw_s[b3][cl * 4];   // (w0 | w1), (w2 | w3)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t p01 = __builtin_amdgcn_perm(xr[1][e >> 1], xr[0][e >> 1], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(xr[3][e >> 1], xr[2][e >> 1], sel);
        float accv = a.conv_b ? bf2f(cb_s[b3][cl]) : 0.f;
        accv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01),
                                              __builtin_bit_cast(bf16x2, wr.x), accv, false);
        accv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23),
                                              __builtin_bit_cast(bf16x2, wr.y), accv, false);
        u[e] = silu_f(accv);
      }
      uint4 hi, lo;
      split_bf2(u[0], u[1], hi.x, lo.x);
      split_bf2(u[2], u[3], hi.y, lo.y);
      split_bf2(u[4], u[5], hi.z, lo.z);
      split_bf2(u[6], u[7], hi.w, lo.w);
      // fragment lane (token % 16) + 16 * grp of column block token / 16
      const int fo = (grp * 16 + (ptok & 15)) * 8;
      *(uint4 *)&u_s[ck & 1][0][ptok >> 4][fo] = hi;
      *(uint4 *)&u_s[ck & 1][1][ptok >> 4][fo] = lo;
    }
  };

  // ---- consumer: wave 8 + cw owns tokens 32 (cw & 3) .. +31 (two MFMA column blocks) and the
  // output blocks of half og = cw >> 2 (blocks og NB0 .. og NB0 + nbn - 1), so every W_x
  // fragment read from LDS feeds four MFMAs
  constexpr int TB = 2;
  constexpr int NB0 = (NB + 1) / 2;              // blocks in the first half (the second: NB - NB0)
  const int cw = wv - 8;
  const int tg = cw & 3, og = cw >> 2;
  const int nb0 = og * NB0, nbn = og ? NB - NB0 : NB0;
  const int tl = lane & 15, g = lane >> 4;
  f32x4 acc[TB][NB0];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int i = 0; i < NB0; ++i) acc[tb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int ck) {
    const int ub = ck & 1, b4 = ck & 3;
    bf16x8 fh[TB], fl[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int cb = tg * TB + tb;
      fh[tb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&u_s[ub][0][cb][lane * 8]);
      fl[tb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&u_s[ub][1][cb][lane * 8]);
    }
#pragma unroll
    for (int i = 0; i < NB0; ++i) {
      if (i < nbn) {   // wave-uniform
        const bf16x8 fw = __builtin_bit_cast(bf16x8, *(const uint4 *)&w_s[b4][nb0 + i][lane * 8]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          acc[tb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fl[tb], acc[tb][i], 0, 0, 0);
          acc[tb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fh[tb], acc[tb][i], 0, 0, 0);
        }
      }
    }
  };

  // The two roles run separate loops with the same barrier count (nck + 1), so the consumers'
  // accumulators are not live in the producers' code; one more barrier (every wave) passes the
  // consumers' partial sums of squares between the two output halves of each token.
  // acc[tb][i][j] = xdbl[token (tg TB + tb) 16 + tl][(nb0 + i) 16 + 4 g + j]; the B | C column
  // of block nb >= RB is (nb - RB) 16 + 4 g (B below N)
  auto bcol = [&](int nb) { return (nb - RB) * 16 + 4 * g; };
  if (producer) {
    issue(0);
    if (nck > 1) issue(1);
    for (int it = 0; it <= nck; ++it) {
      // chunk it's loads (issued two iterations ago) have landed; chunk it+1's may be in flight
      if (it + 1 < nck) {
        if ((it + 1) & 1) wait_vmem_le<PODD>();
        else wait_vmem_le<PEVEN>();
      } else {
        wait_vmem_all();
      }
      lds_barrier();
      if (it + 2 < nck) issue(it + 2);
      if (it < nck) produce(it);
    }
  } else {
    for (int it = 0; it <= nck; ++it) {
      lds_barrier();
      if (it > 0) consume(it - 1);
    }
    // this half's sums of squares of dt_low, B and C per token (the 4 lanes of a token are
    // l % 16 + 16 {0, 1, 2, 3})
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float ssd = 0.f, ssb = 0.f, ssc = 0.f;
#pragma unroll
      for (int i = 0; i < NB0; ++i) {
        if (i < nbn) {
          const int nb = nb0 + i;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = acc[tb][i][j];
            if (nb < RB) ssd = __builtin_fmaf(v, v, ssd);
            else if (bcol(nb) < N) ssb = __builtin_fmaf(v, v, ssb);
            else ssc = __builtin_fmaf(v, v, ssc);
          }
        }
      }
      ssd += __shfl_xor(ssd, 16, 64); ssd += __shfl_xor(ssd, 32, 64);
      ssb += __shfl_xor(ssb, 16, 64); ssb += __shfl_xor(ssb, 32, 64);
      ssc += __shfl_xor(ssc, 16, 64); ssc += __shfl_xor(ssc, 32, 64);
      if (g == 0) *(float4 *)&ss_s[cw][tb * 16 + tl][0] = make_float4(ssd, ssb, ssc, 0.f);
    }
  }
  lds_barrier();
  if (producer) return;

  // ---- epilogue: both halves' sums (first half + second half, the same order in both
  // waves), the three RMSNorms, and this half's outputs
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const float4 s0 = *(const float4 *)&ss_s[tg][tb * 16 + tl][0];
    const float4 s1 = *(const float4 *)&ss_s[tg + 4][tb * 16 + tl][0];
    const float ssd = s0.x + s1.x, ssb = s0.y + s1.y, ssc = s0.z + s1.z;
    const float id = 1.0f / sqrtf(ssd / (float)R + a.eps);
    const float ib = 1.0f / sqrtf(ssb / (float)N + a.eps);
    const float ic = 1.0f / sqrtf(ssc / (float)N + a.eps);
    const int t = t0 + (tg * TB + tb) * 16 + tl;
    if (t < a.L) {
      const int64_t tok = (int64_t)b * a.L + t;
#pragma unroll
      for (int i = 0; i < NB0; ++i) {
        if (i >= nbn) continue;
        const int nb = nb0 + i;
        if (nb < RB) {
          const int n = nb * 16 + 4 * g;
          const float4 gm = *(const float4 *)(a.g_dt + n);
          const float v0 = acc[tb][i][0] * id * gm.x, v1 = acc[tb][i][1] * id * gm.y;
          const float v2 = acc[tb][i][2] * id * gm.z, v3 = acc[tb][i][3] * id * gm.w;
          uint2 h, l;
          split_bf2(v0, v1, h.x, l.x);
          split_bf2(v2, v3, h.y, l.y);
          *(uint2 *)(a.dtlow + tok * R + n) = h;
          *(uint2 *)(a.dtlow_lo + tok * R + n) = l;
        } else {
          const int col = bcol(nb);
          const bool isb = col < N;
          const float4 gm = *(const float4 *)(isb ? a.g_B + col : a.g_C + (col - N));
          const float sc = isb ? ib : ic;
          *(float4 *)(a.bc + tok * (2 * N) + col) =
              make_float4(acc[tb][i][0] * sc * gm.x, acc[tb][i][1] * sc * gm.y,
                          acc[tb][i][2] * sc * gm.z, acc[tb][i][3] * sc * gm.w);
        }
      }
    }
  }
}

template <int RB>
hipError_t launch_rb(const XprojFusedArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * ((a.L + kTok - 1) / kTok));
  if (a.K != 4) return hipErrorInvalidValue;
  switch (a.N) {
    case 8: hipLaunchKernelGGL((xproj_fused_kernel<RB, 4, 8>), dim3(grid), dim3(1024), 0, s, a); break;
    case 16: hipLaunchKernelGGL((xproj_fused_kernel<RB, 4, 16>), dim3(grid), dim3(1024), 0, s, a); break;
    case 32: hipLaunchKernelGGL((xproj_fused_kernel<RB, 4, 32>), dim3(grid), dim3(1024), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// d_state 8 / 16 / 32: R + 2N output rows in whole 16-row blocks, W_x in 4 LDS stages
bool xproj_fused_supported(int R, int N, int D, int K) {
  return (N == 8 || N == 16 || N == 32) && K == 4 && D % (2 * kKC) == 0 &&
         (R == 64 || R == 128 || R == 256);
}

hipError_t launch_xproj_fused(const XprojFusedArgs &a, hipStream_t s) {
  switch (a.R) {
    case 64: return launch_rb<4>(a, s);
    case 128: return launch_rb<8>(a, s);
    case 256: return launch_rb<16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mm
