// Batched single-token decode step (bf16 I/O, fp32 state).
//
// Jamba analysis page, "Inference behavior (generation)": at inference Mamba advances one token
// at a time in O(1): the fixed-size state is updated from the new token with no re-scan. Per
// sequence b and channel i: u = SiLU(conv(conv_state, x_t)), the x_proj / RMSNorm / dt_proj
// chain of the prefill, then h = exp(dt A) h + Bbar u and y = (C . h + D u) SiLU(z)
// ("The Mamba Layer": ZOH and recurrence equations; RMSNorm equation).
//
// Kernels:
//   decode_xproj_kernel  64 sequences x one channel range of d_inner per workgroup (the sequence
//                        tiles of a range on one XCD): u in fp32 from the carried conv state
//                        and x_t (each lane forms exactly its MFMA fragment), split hi + lo,
//                        two bf16 MFMA passes against W_x chunks that stream through
//                        XOR-swizzled LDS (direct-to-LDS loads, double-buffered; a chunk's
//                        global inputs are loaded during the previous chunk's arithmetic).
//                        Writes the range's fp32 partial sums of xdbl.
//   decode_norm_kernel   sums the ranges' partials in a fixed order (deterministic) and applies
//                        the three RMSNorms: dt_low (bf16 hi + lo, for dt_proj) and B | C (fp32);
//                        one thread per value of the sequence for the combine and the norm.
//   decode_update_kernel the state update: 4 lanes per channel, 4 states each as one float4, so
//                        a wave reads / writes 1 KB of state per instruction (the step is
//                        bound by this read-modify-write); conv recomputed; y reduced over the
//                        4 lanes by DPP; the new conv state written in the same pass.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kSeqW = 64;     // sequences per workgroup (4 waves x 16)
constexpr int kKC = 64;       // channels per chunk

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int NX>
__global__ __launch_bounds__(256) void decode_xproj_kernel(DecodeXprojArgs a) {
  constexpr int NB = NX / 16;
  __shared__ __attribute__((aligned(16))) bf16_t w_s0[NX][kKC];
  __shared__ __attribute__((aligned(16))) bf16_t w_s1[NX][kKC];

  const int nseqt = (a.B + kSeqW - 1) / kSeqW;
  // the sequence tiles of one channel range run on one XCD, so that range's W_x rows cross
  // from memory into that XCD's L2 once and serve every tile from there
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int st = gid % nseqt, kr = gid / nseqt;   // sequence tile, channel range
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar load loop
  const int tl = lane & 15, g = lane >> 4;
  const int bs = st * kSeqW + wv * 16 + tl;       // this lane's sequence
  const int bsc = min(bs, a.B - 1);
  const int cbeg = kr * a.range_ch;
  const int nck = min(a.range_ch, a.D - cbeg) / kKC;

  auto stage = [&](int ck, bf16_t (*wdst)[kKC]) {
    const int c0 = cbeg + ck * kKC;
    for (int ld = wv; ld < NX / 8; ld += 4) {
      const int r = ld * 8 + (lane >> 3), ps = lane & 7;
      __builtin_amdgcn_global_load_lds(a.w + (int64_t)r * a.D + c0 + swz(r, ps) * 8,
                                       (__attribute__((address_space(3))) void *)&wdst[ld * 8][0],
                                       16, 0, 0);
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the global inputs of one chunk's two k-steps: carried conv state, x_t, taps and bias
  struct ChunkIn {
    uint4 cs[2][3], x[2], b[2];
    uint2 w[2][8];
  };
  const bf16_t *cbp = a.conv_b ? a.conv_b : a.conv_w;   // without a bias: read, not used
  auto load_in = [&](int ck, ChunkIn &in) {
    const int c0 = cbeg + ck * kKC;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = c0 + (ks * 4 + g) * 8;
      const bf16_t *csp = a.conv_state + ((int64_t)bsc * a.D + ch) * 3;
#pragma unroll
      for (int q = 0; q < 3; ++q) in.cs[ks][q] = *(const uint4 *)(csp + 8 * q);
      in.x[ks] = *(const uint4 *)(a.xz + (int64_t)bsc * 2 * a.D + ch);
#pragma unroll
      for (int e = 0; e < 8; ++e) in.w[ks][e] = *(const uint2 *)(a.conv_w + (int64_t)(ch + e) * 4);
      in.b[ks] = *(const uint4 *)(cbp + ch);   // the 8 channels' bias
    }
  };
  // Chunk ck: its W_x rows and global inputs were issued one chunk earlier, so their latency
  // is hidden behind the previous chunk's arithmetic; the next chunk's are issued before this
  // one's arithmetic. Nothing newer than them is in flight at the wait.
  auto chunk = [&](int ck, const ChunkIn &in, ChunkIn &nxt, bf16_t (*wcur)[kKC],
                   bf16_t (*wnxt)[kKC]) {
    wait_vmem_all();
    lds_barrier();
    if (ck + 1 < nck) {
      stage(ck + 1, wnxt);
      load_in(ck + 1, nxt);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lc = ks * 4 + g;                       // 8 channels: c0 + 8 lc .. +7
      // conv window: carried state (3 per channel, oldest first) then x_t
      const uint4 s0 = in.cs[ks][0], s1 = in.cs[ks][1], s2 = in.cs[ks][2];
      const uint32_t sw[12] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w,
                               s2.x, s2.y, s2.z, s2.w};
      const uint4 xv = in.x[ks];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      float u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint2 wr = in.w[ks][e];
        const uint32_t bw = e < 2 ? in.b[ks].x : e < 4 ? in.b[ks].y : e < 6 ? in.b[ks].z : in.b[ks].w;
        float acc0 = a.conv_b ? ((e & 1) ? hi_bf(bw) : lo_bf(bw)) : 0.f;
        const int s = e * 3;  // bf16 index of channel e's first state value
        const float c0v = (s & 1) ? hi_bf(sw[s >> 1]) : lo_bf(sw[s >> 1]);
        const float c1v = ((s + 1) & 1) ? hi_bf(sw[(s + 1) >> 1]) : lo_bf(sw[(s + 1) >> 1]);
        const float c2v = ((s + 2) & 1) ? hi_bf(sw[(s + 2) >> 1]) : lo_bf(sw[(s + 2) >> 1]);
        const float x = (e & 1) ? hi_bf(xw[e >> 1]) : lo_bf(xw[e >> 1]);
        acc0 = __builtin_fmaf(lo_bf(wr.x), c0v, acc0);
        acc0 = __builtin_fmaf(hi_bf(wr.x), c1v, acc0);
        acc0 = __builtin_fmaf(lo_bf(wr.y), c2v, acc0);
        acc0 = __builtin_fmaf(hi_bf(wr.y), x, acc0);
        u[e] = silu_f(acc0);
      }
      uint4 hi, lo;
      split_bf2(u[0], u[1], hi.x, lo.x);
      split_bf2(u[2], u[3], hi.y, lo.y);
      split_bf2(u[4], u[5], hi.z, lo.z);
      split_bf2(u[6], u[7], hi.w, lo.w);
      const bf16x8 fh = __builtin_bit_cast(bf16x8, hi), fl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + tl;
        const bf16x8 fw = __builtin_bit_cast(bf16x8, *(const uint4 *)&wcur[r][swz(r, lc) * 8]);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fl, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw, fh, acc[nb], 0, 0, 0);
      }
    }
  };

  // two register sets of inputs, alternating with the two W_x buffers
  ChunkIn in0, in1;
  stage(0, w_s0);
  load_in(0, in0);
  for (int ck = 0; ck < nck; ck += 2) {
    chunk(ck, in0, in1, w_s0, w_s1);
    if (ck + 1 < nck) chunk(ck + 1, in1, in0, w_s1, w_s0);
  }
  // partial sums of this channel range: part[kr][b][n]
  if (bs < a.B) {
    float *pp = a.part + ((int64_t)kr * a.B + bs) * NX;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *(float4 *)(pp + nb * 16 + 4 * g) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
  }
}

// One workgroup (16 waves) per sequence: wave w sums ranges w, w + 16, ...; the waves' sums are
// added in a fixed order (deterministic), then wave 0 normalises.
constexpr int kNormWaves = 16;
__global__ __launch_bounds__(64 * kNormWaves) void decode_norm_kernel(DecodeNormArgs a) {
  constexpr int kV = 10;   // NX <= 640 values per sequence over 64 lanes
  __shared__ float red_s[kNormWaves][kV * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const int NX = a.R + 32;
  const int64_t rs = (int64_t)a.B * NX;
  const float *pp = a.part + (int64_t)b * NX;
  float v[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) v[k] = 0.f;
  // loads at a clamped index (always in bounds) and a masked add, so that the loads of a range
  // are issued together rather than each behind its own branch and wait; same order of sums
#pragma unroll 4
  for (int r = wv; r < a.nranges; r += kNormWaves) {
    const float *q = pp + r * rs;
    float x[kV];
#pragma unroll
    for (int k = 0; k < kV; ++k) x[k] = q[min(lane + 64 * k, NX - 1)];
#pragma unroll
    for (int k = 0; k < kV; ++k) v[k] += lane + 64 * k < NX ? x[k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < kV; ++k) red_s[wv][lane + 64 * k] = v[k];
  __syncthreads();
  // thread n combines value n over the waves (fixed order), then the three sums of squares
  // (dt_low over [0, R), B over [R, R+16), C over [R+16, R+32)) are wave sums followed by a
  // fixed-order sum over the waves, and thread n normalises its value
  __shared__ float ss_s[kNormWaves][3];
  const int n = threadIdx.x;
  float s = 0.f;
  if (n < NX) {
#pragma unroll
    for (int w = 0; w < kNormWaves; ++w) s += red_s[w][n];
  }
  const float sq = s * s;
  float pd = n < a.R ? sq : 0.f;
  float pb = (n >= a.R && n < a.R + 16) ? sq : 0.f;
  float pc = (n >= a.R + 16 && n < NX) ? sq : 0.f;
  pd = wave_sum(pd);
  pb = wave_sum(pb);
  pc = wave_sum(pc);
  if (lane == 0) {
    ss_s[wv][0] = pd;
    ss_s[wv][1] = pb;
    ss_s[wv][2] = pc;
  }
  __syncthreads();
  float ssd = 0.f, ssb = 0.f, ssc = 0.f;
#pragma unroll
  for (int w = 0; w < kNormWaves; ++w) {
    ssd += ss_s[w][0];
    ssb += ss_s[w][1];
    ssc += ss_s[w][2];
  }
  const float id = 1.0f / sqrtf(ssd / (float)a.R + a.eps);
  const float ib = 1.0f / sqrtf(ssb / 16.0f + a.eps);
  const float ic = 1.0f / sqrtf(ssc / 16.0f + a.eps);
  if (n < a.R) {
    const float x = s * id * a.g_dt[n];
    a.dtlow[(int64_t)b * a.R + n] = f2bf(x);
    a.dtlow_lo[(int64_t)b * a.R + n] = f2bf(x - bf2f(f2bf(x)));
  } else if (n < a.R + 16) {
    a.bc[(int64_t)b * 32 + (n - a.R)] = s * ib * a.g_B[n - a.R];
  } else if (n < NX) {
    a.bc[(int64_t)b * 32 + (n - a.R)] = s * ic * a.g_C[n - a.R - 16];
  }
}

// State update. With SEQ = false a workgroup covers U x 64 consecutive (b, i) channels; in
// unit j, lane l of a wave takes channel 64 j + l / 4 of its 16-channel slice, states
// 4 (l % 4) .. +3, so each state load / store of a wave is 1 KB contiguous. With SEQ = true a
// workgroup covers 64 channels of U consecutive sequences (unit j = sequence j of the group):
// the channel's A row, taps, bias and D are then loaded once for the U units. The loads of all
// U units are issued before any arithmetic; per-channel scalars are fetched once per channel
// (one lane each) and shared within the channel's 4 lanes by DPP, the sequence's B | C row
// once per wave and shared by bpermute. U = 2 keeps the kernel under 64 VGPRs (the most waves
// per SIMD) with two units of state in flight per lane.
template <bool ZOH, int U, bool SEQ>
__global__ __launch_bounds__(256) void decode_update_kernel(DecodeUpdateArgs a) {
  const int q = threadIdx.x & 3;
  // unit j: (b, i) = gch(j) / D, gch(j) % D
  const int ngc = a.D / 64;
  const int64_t seq0 = SEQ ? (int64_t)(blockIdx.x / ngc) * U : 0;
  const int ich = SEQ ? (int)(blockIdx.x % ngc) * 64 + (threadIdx.x >> 2) : 0;
  const int64_t g0 = SEQ ? seq0 * a.D + ich
                         : (int64_t)blockIdx.x * (64 * U) + (threadIdx.x >> 2);   // b * D + i
  const int64_t w0 = SEQ ? seq0 * a.D : (int64_t)blockIdx.x * (64 * U) + (threadIdx.x >> 6) * 16;
  const int64_t ustep = SEQ ? (int64_t)a.D : 64;   // gch(j + 1) - gch(j)
  float4 h[U], Av[U];
  float Bq[U][4], Cq[U][4];
  uint32_t cs16[U], p16[U];
  float Dv[U], dtv[U];
  uint2 wr[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t gch = g0 + ustep * j;
    const int i = SEQ ? ich : (int)(gch % a.D);
    const int b = SEQ ? (int)seq0 + j : (int)(gch / a.D);
    // the wave's 16 channels of unit j lie in one sequence (d_inner % 16 == 0)
    const int bw = SEQ ? (int)seq0 + j : __builtin_amdgcn_readfirstlane((int)((w0 + 64 * j) / a.D));
    {   // the state streams through once per step: non-temporal, so it does not evict the
        // weights and staged rows the other kernels of the step reuse from L2
      const f32x4 hv4 = __builtin_nontemporal_load((const f32x4 *)(a.state + gch * 16 + 4 * q));
      h[j] = make_float4(hv4[0], hv4[1], hv4[2], hv4[3]);
    }
    if (!SEQ || j == 0) Av[j] = *(const float4 *)(a.A + (int64_t)i * 16 + 4 * q);
    else Av[j] = Av[0];
    // lane l holds value l % 32 of the sequence's B | C row; lanes fetch theirs by bpermute
    const float bcl = a.bc[(int64_t)bw * 32 + (threadIdx.x & 31)];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Bq[j][s] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((4 * q + s) * 4, __builtin_bit_cast(int, bcl)));
      Cq[j][s] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((16 + 4 * q + s) * 4, __builtin_bit_cast(int, bcl)));
    }
    // lane q of the channel loads conv state element min(q, 2); then x | z | - | bias by q
    cs16[j] = a.conv_state[gch * 3 + (q < 3 ? q : 2)];
    const bf16_t *xrow = a.xz + (int64_t)b * 2 * a.D;
    const uint16_t *src = q == 0 ? xrow + i
                        : q == 1 || q == 2 ? xrow + a.D + i
                        : (a.conv_b ? a.conv_b + i : xrow + i);
    p16[j] = *src;
    if (q == 3 && !a.conv_b) p16[j] = 0;
    dtv[j] = a.dt[gch];   // fp32 dt (the channel's 4 lanes read the same word)
    if (!SEQ || j == 0) {
      wr[j] = *(const uint2 *)(a.conv_w + (int64_t)i * 4);
      Dv[j] = a.Dskip[i];
    } else {
      wr[j] = wr[0];
      Dv[j] = Dv[0];
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t gch = g0 + ustep * j;
    const int cs = (int)cs16[j], pv = (int)p16[j];
    const float c0 = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(cs, 0x00, 0xF, 0xF, false));
    const float c1 = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(cs, 0x55, 0xF, 0xF, false));
    const float c2 = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(cs, 0xAA, 0xF, 0xF, false));
    const float xv = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(pv, 0x00, 0xF, 0xF, false));
    const float zv = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(pv, 0x55, 0xF, 0xF, false));
    const float bias = bf2f((bf16_t)__builtin_amdgcn_mov_dpp(pv, 0xFF, 0xF, 0xF, false));
    const float dt = dtv[j];
    float acc = bias;
    acc = __builtin_fmaf(lo_bf(wr[j].x), c0, acc);
    acc = __builtin_fmaf(hi_bf(wr[j].x), c1, acc);
    acc = __builtin_fmaf(lo_bf(wr[j].y), c2, acc);
    acc = __builtin_fmaf(hi_bf(wr[j].y), xv, acc);
    const float u = silu_f(acc);
    const float av[4] = {Av[j].x, Av[j].y, Av[j].z, Av[j].w};
    float hv[4] = {h[j].x, h[j].y, h[j].z, h[j].w};
    float yp = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (ZOH) {
        const float em1 = expm1_f(dt * av[s]);
        hv[s] = __builtin_fmaf(em1 + 1.0f, hv[s], em1 / av[s] * Bq[j][s] * u);
      } else {
        hv[s] = __builtin_fmaf(exp2_hw(dt * av[s] * kLog2e), hv[s], dt * u * Bq[j][s]);
      }
      yp = __builtin_fmaf(Cq[j][s], hv[s], yp);
    }
    __builtin_nontemporal_store(f32x4{hv[0], hv[1], hv[2], hv[3]},
                                (f32x4 *)(a.state + gch * 16 + 4 * q));
    // sum the channel's 4 lanes: quad_perm [1,0,3,2] then [2,3,0,1]
    yp += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, yp), 0xB1, 0xF, 0xF, false));
    yp += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, yp), 0x4E, 0xF, 0xF, false));
    if (q == 0) a.y[gch] = f2bf(__builtin_fmaf(Dv[j], u, yp) * silu_f(zv));
    if (q < 3) a.conv_state[gch * 3 + q] = f2bf(q == 0 ? c1 : q == 1 ? c2 : xv);   // shift in x_t
  }
}

template <int NX>
hipError_t launch_xp(const DecodeXprojArgs &a, hipStream_t s) {
  const int nseqt = (a.B + kSeqW - 1) / kSeqW;
  const int nr = (a.D + a.range_ch - 1) / a.range_ch;
  hipLaunchKernelGGL((decode_xproj_kernel<NX>), dim3((unsigned)(nseqt * nr)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int R, int N, int D, int K) {
  return N == 16 && K == 4 && D % kKC == 0 && (R == 64 || R == 128 || R == 256 || R == 512);
}

hipError_t launch_decode_xproj(const DecodeXprojArgs &a, hipStream_t s) {
  switch (a.R) {
    case 64: return launch_xp<96>(a, s);
    case 128: return launch_xp<160>(a, s);
    case 256: return launch_xp<288>(a, s);
    case 512: return launch_xp<544>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_norm(const DecodeNormArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(decode_norm_kernel, dim3((unsigned)a.B), dim3(64 * kNormWaves), 0, s, a);
  return hipGetLastError();
}

template <bool ZOH>
hipError_t launch_upd(const DecodeUpdateArgs &a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.D;   // a multiple of 64
  if (a.B % 2 == 0)        // pairs of sequences share each channel's parameters
    hipLaunchKernelGGL((decode_update_kernel<ZOH, 2, true>), dim3((unsigned)(n / 128)), dim3(256), 0, s, a);
  else if (n % 128 == 0)
    hipLaunchKernelGGL((decode_update_kernel<ZOH, 2, false>), dim3((unsigned)(n / 128)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_update_kernel<ZOH, 1, false>), dim3((unsigned)(n / 64)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_update(const DecodeUpdateArgs &a, bool zoh, hipStream_t s) {
  return zoh ? launch_upd<true>(a, s) : launch_upd<false>(a, s);
}

}  // namespace mm
