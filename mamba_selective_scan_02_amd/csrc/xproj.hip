// Fused conv1d + SiLU -> x_proj (split-precision bf16 MFMA) -> RMSNorm of dt_low, B, C.
//
// Jamba analysis page: "The selective mechanism" (B, C and Delta from small linear layers of
// the token) and "RMSNorm definition and placement" / "Stabilization: RMSNorm in Mamba layers"
// (RMSNorm on the mixer's internal activations). The conv1d + SiLU producing the projection's
// input is the standard Mamba-1 block the page builds on.
//
// Design (bf16 I/O, dt_rank = 16 * RB, d_state = 16):
//   * One workgroup = 8 waves = a tile of 128 consecutive tokens of one sequence, and ALL
//     R + 2N outputs of those tokens, so every (token, channel) input u is formed once and the
//     three RMSNorms can run in the epilogue (xdbl never goes to memory).
//   * The contraction over d_inner advances in chunks of 64 channels. For each chunk the 131
//     x rows (3 conv-window rows before the tile) and the [R+2N x 64] slice of W_x stream into
//     LDS with direct-to-LDS 16-byte loads, double-buffered so chunk c+1 loads while chunk c
//     is multiplied. Rows are 128 B; 16-byte slot s of row r holds logical chunk s ^ ((r>>1)&7),
//     which makes the 16-row fragment reads of the MFMA loop bank-conflict free.
//   * Lane l of wave w owns token 16w + l%16 and channels 8*(l/16) .. +7 of each 32-channel
//     k-step: exactly the MFMA B-operand fragment of v_mfma_f32_16x16x32_bf16. It computes
//     u = SiLU(conv) for those 8 channels in fp32 from the staged x rows (the 4-tap conv as
//     two packed bf16 dot products per channel), splits
//     u = hi + lo (both bf16) and issues two MFMAs per W fragment, so the product carries u to
//     ~2^-17 relative.
//   * Epilogue: lane (token, 4 consecutive outputs per 16-wide block) squares and sums its
//     dt_low / B / C values, the 4 lanes of a token reduce by lane shuffles, and the normalised
//     dt_low (as bf16 hi + lo for dt_proj) and B|C (fp32) are written.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTok = 128;          // tokens per workgroup
constexpr int kKC = 64;            // channels per chunk
constexpr int kXRowsX = kTok + 8;  // staged x rows: 3 before the tile + 128, padded to 8-row windows

__device__ __forceinline__ void load_lds16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
// physical 16-byte slot of logical chunk c (0..7) in 128-byte row r
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int RB, int K>
__global__ __launch_bounds__(512) void xproj_fused_kernel(XprojFusedArgs a) {
  static_assert(K == 4, "the staged conv taps are laid out as [channel][4]");
  constexpr int R = RB * 16;
  constexpr int NX = R + 32;           // outputs: dt_low | B | C
  constexpr int NB = NX / 16;          // 16-row MFMA blocks
  __shared__ __attribute__((aligned(16))) bf16_t w_s[2][NX][kKC];
  __shared__ __attribute__((aligned(16))) bf16_t x_s[2][kXRowsX][kKC];
  __shared__ __attribute__((aligned(16))) bf16_t cw_s[2][kKC * 4];   // conv taps, [ch][4]
  __shared__ __attribute__((aligned(16))) bf16_t cb_s[2][kKC];       // conv bias

  const int tiles_per_seq = (a.L + kTok - 1) / kTok;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = gid / tiles_per_seq;
  const int t0 = (gid % tiles_per_seq) * kTok;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tl = lane & 15, g = lane >> 4;
  const int tw = wv * 16 + tl;                 // tile-relative token of this lane
  const int64_t row = 2LL * a.D;
  const bf16_t *xzb = a.xz + (int64_t)b * a.L * row;
  const int Lm1 = a.L - 1;
  const int nchunks = a.D / kKC;

  auto stage = [&](int ck, int buf) {
    const int c0 = ck * kKC;
    // W_x rows [NX] x 128 B: 8 rows per 1 KB wave-load
    for (int ld = wv; ld < NX / 8; ld += 8) {
      const int r = ld * 8 + (lane >> 3), ps = lane & 7;
      load_lds16(a.w + (int64_t)r * a.D + c0 + swz(r, ps) * 8, &w_s[buf][ld * 8][0]);
    }
    // x rows: row r <-> token t0 - 3 + r (clamped into the sequence; invalid rows unused)
    for (int ld = wv; ld < kXRowsX / 8; ld += 8) {
      const int r = ld * 8 + (lane >> 3), ps = lane & 7;
      const int t = min(max(t0 - 3 + r, 0), Lm1);
      load_lds16(xzb + (int64_t)t * row + c0 + swz(r, ps) * 8, &x_s[buf][ld * 8][0]);
    }
    // conv taps of the 64 channels: 64 x 4 bf16 = 512 B (lanes 0..31 of wave 1), bias 128 B
    if (wv == 1 && lane < 32) load_lds16(a.conv_w + (int64_t)c0 * K + lane * 8, &cw_s[buf][0]);
    if (wv == 2 && lane < 8 && a.conv_b) load_lds16(a.conv_b + c0 + lane * 8, &cb_s[buf][0]);
  };

  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // conv-state rows before token 0 (only the first tile of a sequence reads them)
  const bool first_tile = t0 == 0;

  stage(0, 0);
  for (int ck = 0; ck < nchunks; ++ck) {
    const int buf = ck & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ck + 1 < nchunks) stage(ck + 1, buf ^ 1);
    const int c0 = ck * kKC;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lc = ks * 4 + g;                  // logical 16-byte chunk = 8 channels
      // x rows tw .. tw+3 of this lane's 8 channels (row tw+3 is the current token), as
      // packed bf16 pairs (dword k holds channels 2k, 2k+1)
      uint32_t xr[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = tw + j;
        const uint4 v = *(const uint4 *)&x_s[buf][r][swz(r, lc) * 8];
        xr[j][0] = v.x; xr[j][1] = v.y; xr[j][2] = v.z; xr[j][3] = v.w;
      }
      if (first_tile && tw < 3) {
        // rows before token 0: carried conv state (oldest first) or zeros
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int t = tw + j - 3;
          if (t < 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              uint32_t w = 0;
              if (a.conv_valid && a.conv_state) {
                const int64_t s0 = ((int64_t)b * a.D + c0 + lc * 8 + 2 * k) * (K - 1) + (K - 1) + t;
                w = (uint32_t)a.conv_state[s0] | ((uint32_t)a.conv_state[s0 + (K - 1)] << 16);
              }
              xr[j][k] = w;
            }
          }
        }
      }
      // conv = (x_{t-3}, x_{t-2}) . (w0, w1) + (x_{t-1}, x_t) . (w2, w3) + b: each pair of
      // window rows of one channel is gathered into one bf16x2 (v_perm) and multiplied with the
      // channel's packed taps (v_dot2, fp32 accumulate)
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cl = lc * 8 + e;
        const uint2 wr = *(const uint2 *)&cw_s[buf][cl * 4];   // (w0 | w1), (w2 | w3)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t p01 = __builtin_amdgcn_perm(xr[1][e >> 1], xr[0][e >> 1], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(xr[3][e >> 1], xr[2][e >> 1], sel);
        float accv = a.conv_b ? bf2f(cb_s[buf][cl]) : 0.f;
        accv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01),
                                              __builtin_bit_cast(bf16x2, wr.x), accv, false);
        accv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23),
                                              __builtin_bit_cast(bf16x2, wr.y), accv, false);
        u[e] = silu_f(accv);
      }
      uint4 hi, lo;
      {
        float l8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) l8[e] = u[e] - bf2f(f2bf(u[e]));
        hi.x = pack_bf2(u[0], u[1]); hi.y = pack_bf2(u[2], u[3]);
        hi.z = pack_bf2(u[4], u[5]); hi.w = pack_bf2(u[6], u[7]);
        lo.x = pack_bf2(l8[0], l8[1]); lo.y = pack_bf2(l8[2], l8[3]);
        lo.z = pack_bf2(l8[4], l8[5]); lo.w = pack_bf2(l8[6], l8[7]);
      }
      const bf16x8 fh = __builtin_bit_cast(bf16x8, hi), fl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + tl;
        const bf16x8 fw = __builtin_bit_cast(bf16x8, *(const uint4 *)&w_s[buf][r][swz(r, lc) * 8]);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fl, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fh, acc[nb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: acc[nb][j] = xdbl[token tw][nb*16 + 4g + j]
  float ssd = 0.f, ssb = 0.f, ssc = 0.f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = acc[nb][j];
      if (nb < RB) ssd = __builtin_fmaf(v, v, ssd);
      else if (nb == RB) ssb = __builtin_fmaf(v, v, ssb);
      else ssc = __builtin_fmaf(v, v, ssc);
    }
  // the 4 lanes of a token are l%16 + 16 * {0, 1, 2, 3}
  ssd += __shfl_xor(ssd, 16, 64); ssd += __shfl_xor(ssd, 32, 64);
  ssb += __shfl_xor(ssb, 16, 64); ssb += __shfl_xor(ssb, 32, 64);
  ssc += __shfl_xor(ssc, 16, 64); ssc += __shfl_xor(ssc, 32, 64);
  const float id = 1.0f / sqrtf(ssd / (float)R + a.eps);
  const float ib = 1.0f / sqrtf(ssb / 16.0f + a.eps);
  const float ic = 1.0f / sqrtf(ssc / 16.0f + a.eps);
  const int t = t0 + tw;
  if (t < a.L) {
    const int64_t tok = (int64_t)b * a.L + t;
#pragma unroll
    for (int nb = 0; nb < RB; ++nb) {
      const int n = nb * 16 + 4 * g;
      const float4 gm = *(const float4 *)(a.g_dt + n);
      const float v0 = acc[nb][0] * id * gm.x, v1 = acc[nb][1] * id * gm.y;
      const float v2 = acc[nb][2] * id * gm.z, v3 = acc[nb][3] * id * gm.w;
      uint2 h, l;
      h.x = pack_bf2(v0, v1); h.y = pack_bf2(v2, v3);
      l.x = pack_bf2(v0 - bf2f(f2bf(v0)), v1 - bf2f(f2bf(v1)));
      l.y = pack_bf2(v2 - bf2f(f2bf(v2)), v3 - bf2f(f2bf(v3)));
      *(uint2 *)(a.dtlow + tok * R + n) = h;
      *(uint2 *)(a.dtlow_lo + tok * R + n) = l;
    }
    {
      const float4 gb = *(const float4 *)(a.g_B + 4 * g);
      const float4 gc = *(const float4 *)(a.g_C + 4 * g);
      *(float4 *)(a.bc + tok * 32 + 4 * g) =
          make_float4(acc[RB][0] * ib * gb.x, acc[RB][1] * ib * gb.y, acc[RB][2] * ib * gb.z,
                      acc[RB][3] * ib * gb.w);
      *(float4 *)(a.bc + tok * 32 + 16 + 4 * g) =
          make_float4(acc[RB + 1][0] * ic * gc.x, acc[RB + 1][1] * ic * gc.y,
                      acc[RB + 1][2] * ic * gc.z, acc[RB + 1][3] * ic * gc.w);
    }
  }
}

template <int RB>
hipError_t launch_rb(const XprojFusedArgs &a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * ((a.L + kTok - 1) / kTok));
  if (a.K != 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL((xproj_fused_kernel<RB, 4>), dim3(grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool xproj_fused_supported(int R, int N, int D, int K) {
  return N == 16 && K == 4 && D % kKC == 0 && (R == 64 || R == 128 || R == 256);
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
