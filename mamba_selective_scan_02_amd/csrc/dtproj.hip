// dt_proj + bias + softplus for bf16 I/O on split-precision bf16 MFMA.
//
//   dt[t, i] = softplus(W_dt[i, :] . dt_low[t, :] + b_i)        (stored as fp32)
//
// Jamba analysis page, "The selective mechanism": Delta is a function of the token through a
// small learned linear layer ("From scalar SSM to vector processing": one Delta per channel).
// Softplus maps it to a positive step (Mamba-1 block).
//
// The contraction is short (dt_rank = 256) and the output wide (d_inner per token), so the
// kernel keeps the token side stationary: a workgroup of 8 waves owns 128 tokens; each wave
// loads the MFMA B-operand fragments of its 16 tokens' dt_low (bf16 high and low parts, whole
// dt_rank) into VGPRs once, then streams the workgroup's channel range through LDS in chunks
// of 64 W_dt rows (direct-to-LDS loads, double-buffered, 16-byte slots XOR-swizzled so the
// 16-row fragment reads are bank-conflict free). Per chunk a wave issues
// (64/16) x (dt_rank/32) x 2 MFMAs and writes 16 tokens x 64 channels of fp32 dt.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kTokD = 128;   // tokens per workgroup
constexpr int kChD = 64;     // channels per chunk

__device__ __forceinline__ void load_lds16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// 16-byte slot swizzle for rows of S slots: 16 consecutive rows read at one logical slot land
// in 16 distinct bank groups (64 banks x 4 B).
template <int S>
__device__ __forceinline__ int swz(int r, int c) {
  if (S == 8) return c ^ ((r >> 1) & 7);
  return c ^ (r & 15);
}

template <int R>
__global__ __launch_bounds__(512) void dtproj_kernel(DtprojArgs a, int ch_per_wg) {
  constexpr int S = R / 8;             // 16-byte slots per W_dt row
  constexpr int KS = R / 32;           // k-steps
  __shared__ __attribute__((aligned(16))) bf16_t w_s0[kChD][R];
  __shared__ __attribute__((aligned(16))) bf16_t w_s1[kChD][R];
  __shared__ __attribute__((aligned(16))) float b_s[2][kChD];   // the chunk's bias, with its rows

  const int ntok = (a.T + kTokD - 1) / kTokD;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = gid % ntok, cg = gid / ntok;      // token tile, channel group
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar load loops
  const int tl = lane & 15, g = lane >> 4;
  const int tok = tt * kTokD + wv * 16 + tl;
  const int tokc = min(tok, a.T - 1);
  const int cbeg = cg * ch_per_wg;
  const int nck = ch_per_wg / kChD;

  // this lane's B-operand fragments: token tok, dt_rank slice [32 ks + 8 g, +8)
  uint4 fh[KS], fl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    fh[ks] = *(const uint4 *)(a.dtlow + (int64_t)tokc * R + ks * 32 + g * 8);
    fl[ks] = *(const uint4 *)(a.dtlow_lo + (int64_t)tokc * R + ks * 32 + g * 8);
  }

  auto stage = [&](int ck, bf16_t (*wdst)[R]) {
    const int c0 = cbeg + ck * kChD;
    constexpr int loads = kChD * S / 64;           // 1 KB wave-loads per chunk
    for (int ld = wv; ld < loads; ld += 8) {
      const int e = ld * 64 + lane;                // 16-byte slot index within the chunk
      const int r = e / S, ps = e % S;
      load_lds16(a.w + (int64_t)(c0 + r) * R + swz<S>(r, ps) * 8, &wdst[0][0] + ld * 512);
    }
    if (wv == 0 && lane < kChD / 4) load_lds16(a.bias + c0 + 4 * lane, &b_s[ck & 1][0]);
  };

  // Outputs of chunk ck are stored at the start of chunk ck+1, after that chunk's wait, so
  // the wait for the staged W_dt rows never has to cover freshly issued stores.
  float4 pend[4];
  int pend_c = -1;
  float *drow = a.dt + (int64_t)tokc * a.D + 4 * g;   // this lane's outputs: + channel
  auto flush = [&]() {
    if (pend_c >= 0 && tok < a.T) {
      float4 *p = (float4 *)(drow + pend_c);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) p[4 * nb] = pend[nb];   // channels + 16 nb
    }
  };
  auto chunk = [&](int ck, bf16_t (*wcur)[R], bf16_t (*wnxt)[R]) {
    wait_vmem_all();   // this chunk's W_dt rows (and older stores) have landed
    lds_barrier();     // ... for every wave; the other buffer is free
    if (ck + 1 < nck) stage(ck + 1, wnxt);
    flush();
    f32x4 acc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // per k-step: the four W_dt fragments are read together, then the low-plane MFMAs of the
    // four accumulators and their high-plane MFMAs (each accumulator still takes low, then
    // high, k-step by k-step), so no MFMA waits on the LDS read or on its own predecessor
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 bh = __builtin_bit_cast(bf16x8, fh[ks]);
      const bf16x8 bl = __builtin_bit_cast(bf16x8, fl[ks]);
      bf16x8 fw[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = nb * 16 + tl;
        fw[nb] = __builtin_bit_cast(bf16x8, *(const uint4 *)&wcur[r][swz<S>(r, ks * 4 + g) * 8]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], bl, acc[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], bh, acc[nb], 0, 0, 0);
    }
    // acc[nb][j] = pre-activation of (token tok, channel c0 + 16 nb + 4 g + j)
    const int c0 = cbeg + ck * kChD;
    const float *bcur = &b_s[ck & 1][0];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const float4 bv = *(const float4 *)(bcur + nb * 16 + 4 * g);
      pend[nb] = make_float4(softplus_sel(acc[nb][0] + bv.x), softplus_sel(acc[nb][1] + bv.y),
                             softplus_sel(acc[nb][2] + bv.z), softplus_sel(acc[nb][3] + bv.w));
    }
    pend_c = c0;
  };

  stage(0, w_s0);
  for (int ck = 0; ck < nck; ++ck) {
    const bool odd = ck & 1;
    chunk(ck, odd ? w_s1 : w_s0, odd ? w_s0 : w_s1);
  }
  flush();
}

template <int R>
hipError_t launch_r(const DtprojArgs &a, hipStream_t s) {
  const int ntok = (a.T + kTokD - 1) / kTokD;
  // split the channels so that there are >= 2 workgroups per CU when tokens are few
  int split = 1;
  while (ntok * split < 512 && a.D / (split * 2) >= kChD && (a.D / (split * 2)) % kChD == 0) split *= 2;
  hipLaunchKernelGGL((dtproj_kernel<R>), dim3((unsigned)(ntok * split)), dim3(512), 0, s, a,
                     a.D / split);
  return hipGetLastError();
}

}  // namespace

bool dtproj_supported(int R, int D) {
  return D % kChD == 0 && (R == 64 || R == 128 || R == 256 || R == 512);
}

hipError_t launch_dtproj_tiled(const DtprojArgs &a, hipStream_t s) {
  switch (a.R) {
    case 64: return launch_r<64>(a, s);
    case 128: return launch_r<128>(a, s);
    case 256: return launch_r<256>(a, s);
    case 512: return launch_r<512>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mm
