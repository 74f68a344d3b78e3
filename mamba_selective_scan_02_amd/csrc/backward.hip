// Backward of the mixer prefill: gradients of sum(dy * y) with respect to xz, the parameters
// and the carried states (training through the parallel scan, Jamba analysis page, "Parallel
// training via the parallel scan"). Arithmetic is fp32; xz, dy and dxz are in the I/O dtype.
//
// The forward (continuous SSM / ZOH / recurrence equations of "The Mamba Layer", the RMSNorm
// equation, and the Mamba-1 conv, softplus and gate) is differentiated step by step in reverse:
//   gate      y = ys SiLU(z), ys = C.h + D u  ->  dys = dy SiLU(z), dz = dy ys SiLU'(z)
//   scan      h_t = a_t h_{t-1} + bb_t u_t, a = exp(dt A), bb = dt B (or expm1(dt A) / A B)
//             dh_t = C_t dys_t + a_{t+1} dh_{t+1}, and from dh_t, h_{t-1}: d dt, dA, dB, du
//   softplus  dt = softplus(p)  ->  dp = d dt sigmoid(p)
//   RMSNorm   o = v / r g  ->  dv = g do / r - v sum(g do v) / (n r^3),  dg = sum_t do v / r
//   x_proj / dt_proj: products with the weights (and their transposes); conv + SiLU last.
//
// Kernels, in launch order:
//   bw_conv_u_kernel          u = SiLU(conv1d(x) + b) in fp32                  [T, D]
//   products                  x_proj, dt_proj, their input and weight gradients: with bf16
//                             I/O split-bf16 MFMA products (bwgemm.hip: each fp32 operand as
//                             bf16 high + low planes); with fp32 I/O gemm_f32_kernel (fp32
//                             16x16x4 MFMA, 128 x 128 or 128 x 64 tiles, any strides)
//   (norm_kernel)             the forward's RMSNorm of dt_low, B, C (fp32 mode)
//   bw_range_transfer_kernel  per range of kRT tokens and (channel, 4 states), 64 channels per
//                             workgroup with staged inputs, one forward pass: the forward
//                             transfer (prod a, local end state) and the reverse one (local
//                             a_t0 dh_t0 from zero). The staging forms dt = softplus(p) and
//                             dys = dy SiLU(z) from dt_proj's product, dy and z, once per
//                             (token, channel); neither goes to memory
//   bw_range_carry_kernel     sequential over ranges: each range's true start state and the
//                             dh carry entering it from later ranges; the last carry is the
//                             gradient of the carried SSM state
//   bw_scan_kernel            per range, 32 channels x 16 states per workgroup: a forward pass
//                             (ys = C.h + D u, and the gate's dz = dy ys SiLU'(z) straight to
//                             dxz; checkpoints every kSB2 tokens in LDS), then sub-blocks in
//                             reverse, each recomputed into registers and walked backward,
//                             writing d(dt_proj pre-activation) = d dt sigmoid(p) and du. Each
//                             sub-block's inputs are staged in LDS by coalesced loads issued one
//                             sub-block ahead (the recurrence never waits on global memory).
//                             Sums over the 16 states: transposed DPP reductions within a
//                             16-lane row; dB and dC (shared by all channels) sum over the
//                             wave's 4 channels with lane swaps across rows, over the 8 waves
//                             in LDS, into per-workgroup rows
//   bw_rowsum_kernel          dB | dC from those per-workgroup rows
//   bw_norm_bwd_kernel        the three RMSNorm backwards per token (+ gain terms)
//   bw_colsum_kernels         fixed-order column sums (bias, gains, D, A, conv partials)
//   bw_conv_bwd_kernel        SiLU' and the transposed depthwise convolution in one pass
//                             (sliding windows of x and dq per 64-token strip), conv weight
//                             partials; bw_conv_scatter_kernel places their column sums
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRT = 256;          // tokens per range (carry granularity)
constexpr int kCG = 64;           // channels per scan workgroup
constexpr int kColRows = 1024;    // rows per partial of a column sum

__device__ __forceinline__ float sigmoid_f(float v) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_hw(-v * kLog2e));
}
__device__ __forceinline__ float dsilu_f(float v) {
  const float s = sigmoid_f(v);
  return s * __builtin_fmaf(v, 1.0f - s, 1.0f);
}
// ---------------------------------------------------------------- weights to fp32
template <typename T>
__global__ __launch_bounds__(256) void to_f32_kernel(const T *src, float *dst, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = io<T>::ld(src + i);
}

// ---------------------------------------------------------------- u = SiLU(conv1d(x) + b)
// x at position s < 0 is the carried conv state (index K-1+s, oldest first) or zero.
template <typename T>
__device__ __forceinline__ float conv_in(const BwArgs &a, int b, int s, int i) {
  if (s >= 0) return io<T>::ld((const T *)a.xz + ((int64_t)b * a.L + s) * 2 * a.D + i);
  if (!a.cs_valid) return 0.f;
  return io<T>::ld((const T *)a.conv_state + ((int64_t)b * a.D + i) * (a.K - 1) + (a.K - 1 + s));
}
template <typename T>
__device__ __forceinline__ float conv_pre(const BwArgs &a, int b, int t, int i) {
  float q = a.conv_b ? io<T>::ld((const T *)a.conv_b + i) : 0.f;
  for (int k = 0; k < a.K; ++k)
    q = __builtin_fmaf(io<T>::ld((const T *)a.conv_w + i * a.K + k), conv_in<T>(a, b, t - (a.K - 1) + k, i), q);
  return q;
}
// 4 consecutive channels of a row (8-byte bf16 / 16-byte fp32 accesses)
template <typename T> struct v4io;
template <> struct v4io<float> {
  static __device__ __forceinline__ void ld(const float *p, float v[4]) {
    const float4 x = *(const float4 *)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  static __device__ __forceinline__ void st(float *p, const float v[4]) {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct v4io<bf16_t> {
  static __device__ __forceinline__ void ld(const bf16_t *p, float v[4]) {
    const uint2 x = *(const uint2 *)p;
    v[0] = lo_bf(x.x); v[1] = hi_bf(x.x); v[2] = lo_bf(x.y); v[3] = hi_bf(x.y);
  }
  static __device__ __forceinline__ void st(bf16_t *p, const float v[4]) {
    uint2 x;
    x.x = pack_bf2(v[0], v[1]);
    x.y = pack_bf2(v[2], v[3]);
    *(uint2 *)p = x;
  }
};
// x of channels i0 .. i0+3 at position s of sequence b (s < 0: the carried state or zero)
template <typename T>
__device__ __forceinline__ void conv_in4(const BwArgs &a, int b, int s, int i0, float v[4]) {
  if (s >= 0) {
    v4io<T>::ld((const T *)a.xz + ((int64_t)b * a.L + s) * 2 * a.D + i0, v);
    return;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = conv_in<T>(a, b, s, i0 + c);
}
// bf16 hi = bf16(v), lo = bf16(v - hi) of 4 values, packed for two 8-byte stores
__device__ __forceinline__ void split4(const float v[4], uint2 &hi, uint2 &lo) {
  bf16_t h[4], l[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    h[c] = f2bf(v[c]);
    l[c] = f2bf(v[c] - bf2f(h[c]));
  }
  hi = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  lo = make_uint2((uint32_t)l[0] | ((uint32_t)l[1] << 16), (uint32_t)l[2] | ((uint32_t)l[3] << 16));
}

// One thread per 4 channels of a kUStrip-token strip (blockIdx.x: strips, blockIdx.y: blocks
// of 1024 channels): the K-tap window slides along the strip, so each x row is read once.
// With u_hi set, u is also written as bf16 hi / lo planes (the split products' operand).
constexpr int kUStrip = 64;
template <typename T, int K>
__global__ __launch_bounds__(256) void bw_conv_u_kernel(BwArgs a) {
  const int i0 = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (i0 >= a.D) return;
  const int ns = (a.L + kUStrip - 1) / kUStrip;
  const int b = blockIdx.x / ns, s0 = (blockIdx.x % ns) * kUStrip;
  const int s1 = min(a.L, s0 + kUStrip);
  float w[4][K], bias[4], xw[K][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    bias[c] = a.conv_b ? io<T>::ld((const T *)a.conv_b + i0 + c) : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) w[c][k] = io<T>::ld((const T *)a.conv_w + (i0 + c) * K + k);
  }
#pragma unroll
  for (int k = 0; k < K - 1; ++k) conv_in4<T>(a, b, s0 - (K - 1) + k, i0, xw[k]);
  for (int t = s0; t < s1; ++t) {
    v4io<T>::ld((const T *)a.xz + ((int64_t)b * a.L + t) * 2 * a.D + i0, xw[K - 1]);
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float q = bias[c];
#pragma unroll
      for (int k = 0; k < K; ++k) q = __builtin_fmaf(w[c][k], xw[k][c], q);
      u[c] = silu_f(q);
    }
    const int64_t e = ((int64_t)b * a.L + t) * a.D + i0;
    v4io<float>::st(a.u + e, u);
    if (a.u_hi) {
      uint2 hi, lo;
      split4(u, hi, lo);
      *(uint2 *)(a.u_hi + e) = hi;
      *(uint2 *)(a.u_lo + e) = lo;
    }
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) xw[k][c] = xw[k + 1][c];
  }
}

// expm1 as expm1_f computes it (hardware exp above |x| = 0.5, Taylor series to x^8 below),
// with both branches evaluated and one selected, so that an unrolled loop needs no divergent
// control flow
__device__ __forceinline__ float expm1_sel(float x) {
  const float big = exp2_hw(x * kLog2e) - 1.0f;
  float r = __builtin_fmaf(x, 1.0f / 8.0f, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 7.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 6.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 5.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 4.0f), r, 1.0f);
  r = __builtin_fmaf(x * (1.0f / 3.0f), r, 1.0f);
  r = __builtin_fmaf(x * 0.5f, r, 1.0f);
  return fabsf(x) > 0.5f ? big : x * r;
}

// ---------------------------------------------------------------- per-range transfers
// One workgroup per range of one sequence and 64 channels. The
// inputs of each kRS-token sub-block (dt, u, dys of the 64 channels: whole 256-byte rows; B|C)
// are staged in LDS by coalesced loads, the next sub-block's fetched into registers while the
// current one is processed. Without ZOH the u slot is staged as dt u.
//
// One forward pass gives all three transfers of the range [t0, t1): P = prod a_t, the local
// end state S (from zero), and the reverse carry R = sum_t (a_t0 ... a_t) C_t dys_t, which is
// the reverse recursion g <- a_t (C_t dys_t + g) from zero at t1 unrolled (the running product
// is P's own). Tokens past t1 are staged as zeros: a = 1 and zero inputs leave all three as
// they are.
// Lanes: 64 channels x 4 groups of 4 states per workgroup (256 threads): the per-(token,
// channel) values are read once per 4 states, and B, C as 16-byte vectors.
constexpr int kRS = 16;                          // tokens per staged sub-block
constexpr int kRA = kRS * kCG;                   // floats per staged [kRS][64] array
static_assert(kRA == 4 * 256 && kRS * 32 == 2 * 256, "four staged elements per thread, two of B|C");
template <typename T, bool ZOH>
__global__ __launch_bounds__(256) void bw_range_transfer_kernel(BwArgs a) {
  __shared__ __attribute__((aligned(16))) float st_s[3 * kRA + kRS * 32];   // dt | dt u (or u) | dys | B|C
  const int ncg = a.D / kCG;
  const int cg = blockIdx.x % ncg;
  const int r = (blockIdx.x / ncg) % a.nr;
  const int b = blockIdx.x / (ncg * a.nr);
  const int tid = threadIdx.x;
  const int sg = tid & 3, c = tid >> 2, i = cg * kCG + c;
  const int t0 = r * kRT, t1 = min(a.L, t0 + kRT);
  const int nsb = (t1 - t0 + kRS - 1) / kRS;
  const int64_t tb = (int64_t)b * a.L;
  const float4 A4 = *(const float4 *)(a.A + i * 16 + 4 * sg);
  const float An[4] = {A4.x, A4.y, A4.z, A4.w};
  float An2[4], rA[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    An2[j] = An[j] * kLog2e;
    rA[j] = ZOH ? 1.0f / An[j] : 0.f;   // ZOH: (e^(dt A) - 1) / A as expm1 times 1 / A
  }
  // this thread stages elements tid + 256 h (token (tid >> 6) + 4 h, channel tid & 63) of the
  // [kRS][64] arrays, h < 4, and of the [kRS][32] B|C array, h < 2
  const int sch = tid & 63;
  const float sbias = a.dt_b[cg * kCG + sch];
  // dy and z stay in the I/O type until the stash: converting them where they are fetched
  // would wait for the loads there, one sub-block too early
  float pp[4], pu[4], pbc[2];
  T rdy[4], rz[4];
  bool pl[4];   // the element's token lies inside the range
  auto fetch = [&](int j) {
    const int tj = t0 + j * kRS;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int k = (tid >> 6) + 4 * h;
      pp[h] = pu[h] = 0.f;
      rdy[h] = rz[h] = T(0);
      pl[h] = tj + k < t1;
      if (pl[h]) {
        const int64_t tok = tb + tj + k, e = tok * a.D + cg * kCG + sch;
        pp[h] = a.dt[e];
        pu[h] = a.u[e];
        rdy[h] = ((const T *)a.dy)[e];
        rz[h] = ((const T *)a.xz)[tok * 2 * a.D + a.D + cg * kCG + sch];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = tid + 256 * h, k = e >> 5;
      pbc[h] = tj + k < t1 ? a.bc[(tb + tj + k) * 32 + (e & 31)] : 0.f;
    }
  };
  // dt = softplus(p), p = product + bias; dys = dy SiLU(z); without ZOH the u slot holds dt u.
  // A token past the range end gets dt = 0: an identity step.
  auto stash = [&]() {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float dt = pl[h] ? softplus_f(pp[h] + sbias) : 0.f;
      st_s[tid + 256 * h] = dt;
      st_s[kRA + tid + 256 * h] = ZOH ? pu[h] : dt * pu[h];
      st_s[2 * kRA + tid + 256 * h] = io<T>::cvt(rdy[h]) * silu_f(io<T>::cvt(rz[h]));
    }
    st_s[3 * kRA + tid] = pbc[0];
    st_s[3 * kRA + 256 + tid] = pbc[1];
  };
  const float *s_dt = st_s, *s_u = st_s + kRA, *s_dys = st_s + 2 * kRA, *s_bc = st_s + 3 * kRA;

  float P[4] = {1.f, 1.f, 1.f, 1.f}, S[4] = {0.f, 0.f, 0.f, 0.f}, g[4] = {0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int j = 0; j < nsb; ++j) {
    __syncthreads();
    stash();
    __syncthreads();
    if (j + 1 < nsb) fetch(j + 1);
#pragma unroll
    for (int k = 0; k < kRS; ++k) {
      const float dtv = s_dt[k * kCG + c], uv = s_u[k * kCG + c], dysv = s_dys[k * kCG + c];
      const float4 B4 = *(const float4 *)&s_bc[k * 32 + 4 * sg];
      const float4 C4 = *(const float4 *)&s_bc[k * 32 + 16 + 4 * sg];
      const float Bv[4] = {B4.x, B4.y, B4.z, B4.w}, Cv[4] = {C4.x, C4.y, C4.z, C4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float av = exp2_hw(dtv * An2[q]);
        const float bu = ZOH ? expm1_sel(dtv * An[q]) * rA[q] * Bv[q] * uv : uv * Bv[q];
        S[q] = __builtin_fmaf(av, S[q], bu);
        P[q] *= av;
        g[q] = __builtin_fmaf(P[q], Cv[q] * dysv, g[q]);
      }
    }
  }
  const int64_t o = (((int64_t)b * a.nr + r) * a.D + i) * 16 + 4 * sg;
  *(float4 *)(a.rP + o) = make_float4(P[0], P[1], P[2], P[3]);
  *(float4 *)(a.rS + o) = make_float4(S[0], S[1], S[2], S[3]);
  *(float4 *)(a.rR + o) = make_float4(g[0], g[1], g[2], g[3]);
}

// sequential over the ranges of one (sequence, channel, state): rS becomes the start state
// of each range, rR the carry a_{t1} dh_{t1} entering it from the ranges after it
__global__ __launch_bounds__(256) void bw_range_carry_kernel(BwArgs a) {
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= (int64_t)a.B * a.D * 16) return;
  const int64_t b = e / ((int64_t)a.D * 16), in = e % ((int64_t)a.D * 16);
  float h = (a.ss_valid && a.ssm_state) ? a.ssm_state[e] : 0.f;
  for (int r = 0; r < a.nr; ++r) {
    const int64_t o = (b * a.nr + r) * a.D * 16 + in;
    const float s = a.rS[o];
    a.rS[o] = h;
    h = __builtin_fmaf(a.rP[o], h, s);
  }
  float g = 0.f;
  for (int r = a.nr - 1; r >= 0; --r) {
    const int64_t o = (b * a.nr + r) * a.D * 16 + in;
    const float rr = a.rR[o];
    a.rR[o] = g;
    g = __builtin_fmaf(a.rP[o], g, rr);
  }
  if (a.d_ssm_state) a.d_ssm_state[e] = g;
}

// ---------------------------------------------------------------- the reverse scan
// Lanes: 32 channels x 16 states per workgroup (512 threads; lane n = state, the wave's four
// 16-lane rows = four channels); one range of one sequence, in sub-blocks of kSB2 tokens whose
// inputs are staged in LDS by coalesced loads one sub-block ahead (per-(token, channel) arrays
// [kSB2][32] and B|C [kSB2][32]; thread tid stages element tid of each). Tokens past the range
// end are staged as zeros (a = 1, no input: the states and the carry pass through them
// unchanged, and nothing of theirs is stored).
//
// Sums over the 16 states of a channel (ys, and the d dt, du contributions) are transposed
// reductions: each lane holds 8 partial values (8 tokens, or 4 tokens x 2 quantities), and
// four DPP exchange-and-add steps inside the row leave lanes 2j and 2j + 1 with the row's sum of
// value j, 22 VALU operations for 8 sums. Sums over the wave's four channels (dB, dC: per token
// and state) are transposed too, across rows, with the lane-swap instructions: a 32-lane swap
// of (dB term, dC term) plus an add leaves rows 0-1 with dB and rows 2-3 with dC summed over
// channel pairs; a 16-lane swap of two tokens' results plus an add finishes both tokens, row r
// holding dB (r = 0, 1) or dC (r = 2, 3) of token 2p + (r & 1). Three swaps and three adds per
// two tokens; each wave's sums go to LDS once per sub-block and the 8 waves are added in a fixed
// order.
constexpr int kSB2 = 16;                        // tokens per recomputed sub-block
constexpr int kNSB2 = kRT / kSB2;               // sub-blocks per range
constexpr int kCG2 = 32;                        // channels per reverse-scan workgroup
constexpr int kST2 = kCG2 * 16;                 // threads: (channel, state)
constexpr int kW2 = kST2 / 64;                  // waves
constexpr int kSF2 = kSB2 * kCG2;               // floats per staged [kSB2][32] array
// staged arrays: dt | u | dt u | dys | sigmoid(p) | dy SiLU'(z) | B|C, one element each
constexpr int kS2NA = 7;
static_assert(kSF2 == kST2 && kSB2 * 32 == kST2, "one staged element per thread and array");

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// v[0..7] in every lane of a 16-lane row -> lane n returns the row's sum of v[n >> 1]. Steps 1-3
// pair lanes that differ in bit 3, 2, 1 of n (row_ror:8, half-row mirror, quad xor 2): each lane
// keeps the half of the remaining values its bit selects and adds the partner's copy of them;
// the last step adds the two copies of the one value left (quad xor 1). 22 VALU operations.
__device__ __forceinline__ float tsum8(const float (&v)[8], int n) {
  const bool b3 = n & 8, b2 = n & 4, b1 = n & 2;
  float w[4], x[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = (b3 ? v[j + 4] : v[j]) + dpp_f<0x128>(b3 ? v[j] : v[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) x[j] = (b2 ? w[j + 2] : w[j]) + dpp_f<0x141>(b2 ? w[j] : w[j + 2]);
  const float y = (b1 ? x[1] : x[0]) + dpp_f<0x4E>(b1 ? x[0] : x[1]);
  return y + dpp_f<0xB1>(y);
}

template <typename T, bool ZOH>
__global__ __launch_bounds__(kST2, 4) void bw_scan_kernel(BwArgs a) {
  __shared__ float ck_s[kNSB2][kST2];       // state checkpoints, one column per thread
  __shared__ float red_s[kW2][kSB2 / 2][64];  // per wave and token pair: dB | dC sums
  __shared__ float st_s[kS2NA * kST2];      // the current sub-block's inputs
  __shared__ float o_s[2][kSB2][kCG2];      // the current sub-block's per-(token, channel) outputs

  const int ncg = a.D / kCG2;
  const int cg = blockIdx.x % ncg;
  const int r = (blockIdx.x / ncg) % a.nr;
  const int b = blockIdx.x / (ncg * a.nr);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, cl = lane >> 4;
  const int c = wv * 4 + cl;                // channel within the group
  const int i = cg * kCG2 + c;
  const int t0 = r * kRT, t1 = min(a.L, t0 + kRT);
  const int nsb = (t1 - t0 + kSB2 - 1) / kSB2;
  const float An = a.A[i * 16 + n], An2 = An * kLog2e;
  const float rA = ZOH ? 1.0f / An : 0.f;   // ZOH: (e^(dt A) - 1) / A as expm1 times 1 / A
  const float Dv = a.Dskip[i];
  const int64_t so = (((int64_t)b * a.nr + r) * a.D + i) * 16 + n;
  const int64_t tb = (int64_t)b * a.L;
  // this thread stages element tid of each array: token tid / 32, channel tid % 32
  const int sk = tid >> 5, sch = tid & 31;
  const float sbias = a.dt_b[cg * kCG2 + sch];
  float pp, pu, pbc;            // dt_proj's product (pre-bias), u; B|C
  T rdy, rz;                    // dy, z in the I/O type (converted at the stash, not at the fetch)
  float dDs = 0.f;              // sum over the range of dys u of this thread's staged column
  bool pl;                      // the element's token lies inside the range
  auto fetch = [&](int j) {
    const int64_t tok = tb + t0 + j * kSB2 + sk, e = tok * a.D + cg * kCG2 + sch;
    pl = t0 + j * kSB2 + sk < t1;
    pp = pu = pbc = 0.f;
    rdy = rz = T(0);
    if (pl) {
      pp = a.dt[e];
      pu = a.u[e];
      rdy = ((const T *)a.dy)[e];
      rz = ((const T *)a.xz)[tok * 2 * a.D + a.D + cg * kCG2 + sch];
      pbc = a.bc[tok * 32 + sch];
    }
  };
  // dt = softplus(p) and sigmoid(p), p = product + bias; dys = dy SiLU(z); dy SiLU'(z) for the
  // gate's dz. A token past the range end gets dt = 0 and no inputs: an identity step.
  // (the forward pass needs dy SiLU'(z), the reverse pass dys and sigmoid(p))
  auto stash = [&](bool rev) {
    const float p = pp + sbias;
    const float pdy = io<T>::cvt(rdy), pz = io<T>::cvt(rz);
    const float dt = pl ? softplus_f(p) : 0.f;
    st_s[tid] = dt;
    st_s[kST2 + tid] = pu;
    st_s[2 * kST2 + tid] = dt * pu;
    if (rev) {
      const float dys = pdy * silu_f(pz);
      st_s[3 * kST2 + tid] = dys;
      st_s[4 * kST2 + tid] = sigmoid_f(p);
      dDs = __builtin_fmaf(dys, pu, dDs);
    } else {
      st_s[5 * kST2 + tid] = pdy * dsilu_f(pz);
    }
    st_s[6 * kST2 + tid] = pbc;
  };
  // per-sub-block output tiles [kSB2][32], written by the lanes that own the sums and stored
  // by one thread per element (whole rows of the 32 channels)
  auto flush_dz = [&](int jp) {   // the forward pass's dz of sub-block jp
    const int t = t0 + jp * kSB2 + sk;
    if (t < t1)
      io<T>::st((T *)a.dxz + (tb + t) * 2 * a.D + a.D + cg * kCG2 + sch, o_s[0][sk][sch]);
  };
  auto flush_dp_du = [&](int jp) {   // the reverse pass's d(dt_proj pre-activation) and du
    const int t = t0 + jp * kSB2 + sk;
    if (t < t1) {
      const int64_t e = (tb + t) * a.D + cg * kCG2 + sch;
      const float dp = o_s[0][sk][sch];
      a.sig[e] = dp;
      if (a.dp_hi) {
        const bf16_t hi = f2bf(dp);
        a.dp_hi[e] = hi;
        a.dp_lo[e] = f2bf(dp - bf2f(hi));
      }
      a.du[e] = o_s[1][sk][sch];
    }
  };
  const float *s_dt = st_s, *s_u = st_s + kST2, *s_dtu = st_s + 2 * kST2,
              *s_dys = st_s + 3 * kST2, *s_sg = st_s + 4 * kST2, *s_gz = st_s + 5 * kST2,
              *s_bc = st_s + 6 * kST2;
  // input contribution of token k to the state: bb_t u_t
  auto bu_of = [&](int k, float dtv) {
    if (ZOH) return expm1_sel(dtv * An) * rA * s_bc[k * 32 + n] * s_u[k * kCG2 + c];
    return s_dtu[k * kCG2 + c] * s_bc[k * 32 + n];
  };

  // pass 1: true states from the range's start state; checkpoints; ys = C.h + D u for the gate
  float h = a.rS[so];
  fetch(0);
  for (int j = 0; j < nsb; ++j) {
    lds_barrier();
    stash(false);
    if (j > 0) flush_dz(j - 1);
    lds_barrier();
    if (j + 1 < nsb) fetch(j + 1);
    ck_s[j][tid] = h;
    float yp[8];
#pragma unroll
    for (int k = 0; k < kSB2; ++k) {
      const float dtv = s_dt[k * kCG2 + c];
      h = __builtin_fmaf(exp2_hw(dtv * An2), h, bu_of(k, dtv));
      yp[k & 7] = s_bc[k * 32 + 16 + n] * h;
      if ((k & 7) == 7) {
        const float ys = tsum8(yp, n);       // token k - 7 + n / 2 (both lanes of a pair)
        const int kt = k - 7 + (n >> 1);
        if (!(n & 1)) {   // the gate: dz = dy ys SiLU'(z), ys = C.h + D u
          const float yv = __builtin_fmaf(Dv, s_u[kt * kCG2 + c], ys);
          o_s[0][kt][c] = s_gz[kt * kCG2 + c] * yv;
        }
      }
    }
  }

  // pass 2: sub-blocks in reverse; carry = a_{t+1} dh_{t+1}
  float carry = a.rR[so];
  float dA = 0.f;
  fetch(nsb - 1);
  for (int j = nsb - 1; j >= 0; --j) {
    lds_barrier();     // the stage, red_s and o_s are free (previous sub-block consumed)
    if (j == nsb - 1) flush_dz(j);   // the forward pass's last tile
    stash(true);
    lds_barrier();
    if (j > 0) fetch(j - 1);
    const int tj = t0 + j * kSB2;
    float rr[kSB2 / 2], sodd = 0.f;          // per token pair: the wave's dB | dC sums
    // window of 4 tokens: with Euler Bbar the two per-state terms whose sums over the states
    // give d dt = sum(ra A) + u sum(dh B) and du = dt sum(dh B) + D dys; with ZOH the d dt and
    // du terms themselves
    float gv[8];
    float hist[kSB2 + 1], ah[kSB2];
    hist[0] = ck_s[j][tid];
#pragma unroll
    for (int k = 0; k < kSB2; ++k) {
      const float dtv = s_dt[k * kCG2 + c];
      ah[k] = exp2_hw(dtv * An2);
      hist[k + 1] = __builtin_fmaf(ah[k], hist[k], bu_of(k, dtv));
    }
    // reverse walk
#pragma unroll
    for (int k = kSB2 - 1; k >= 0; --k) {
      const float dtv = s_dt[k * kCG2 + c], uv = s_u[k * kCG2 + c];
      const float Bn = s_bc[k * 32 + n], Cn = s_bc[k * 32 + 16 + n];
      const float dysv = s_dys[k * kCG2 + c];
      const float av = ah[k];
      const float dh = __builtin_fmaf(Cn, dysv, carry);
      const float ra = dh * hist[k] * av;      // d / d a_t, times a_t
      float pB, g0, g1;
      if (ZOH) {
        const float x = dtv * An;
        const float E = expm1_sel(x), q = E * rA;
        const float dBb = dh * uv;
        g0 = ra * An + dBb * av * Bn;          // d dt
        dA += ra * dtv + dBb * Bn * (x * av - E) * rA * rA;
        pB = dBb * q;
        g1 = dh * q * Bn;                      // du
      } else {
        g0 = ra * An;
        g1 = dh * Bn;
        dA = __builtin_fmaf(ra, dtv, dA);
        pB = dh * s_dtu[k * kCG2 + c];
      }
      const float pC = dysv * hist[k + 1];
      carry = av * dh;
      {
        // rows 0-1: dB terms of channels (0 + 2), (1 + 3); rows 2-3: dC terms likewise
        const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(pB), __float_as_uint(pC),
                                                        false, false);
        const float sk = __uint_as_float(w[0]) + __uint_as_float(w[1]);
        if (k & 1) {
          sodd = sk;
        } else {
          // rows of (token k, token k + 1): dB k | dB k+1 | dC k | dC k+1
          const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(sk),
                                                          __float_as_uint(sodd), false, false);
          rr[k >> 1] = __uint_as_float(v[0]) + __uint_as_float(v[1]);
        }
      }
      gv[k & 3] = g0;
      gv[4 + (k & 3)] = g1;
      if ((k & 3) == 0) {
        // lane n: the sum of g0 (n < 8) or g1 (n >= 8) of token k + (n / 2) % 4 (both lanes of
        // a pair); row_ror:8 hands lane n < 8 the g1 sum of the same token
        const float sv = tsum8(gv, n);
        const int kt = k + ((n >> 1) & 3);
        const float s1 = dpp_f<0x128>(sv);
        if (!(n & 1)) {
          const float dysk = s_dys[kt * kCG2 + c];
          if (ZOH) {
            if (n < 8) o_s[0][kt][c] = sv * s_sg[kt * kCG2 + c];   // d dt sigmoid(p)
            else o_s[1][kt][c] = __builtin_fmaf(Dv, dysk, sv);    // with D u's term
          } else if (n < 8) {
            o_s[0][kt][c] = __builtin_fmaf(s_u[kt * kCG2 + c], s1, sv) * s_sg[kt * kCG2 + c];
          } else {
            o_s[1][kt][c] = __builtin_fmaf(s_dt[kt * kCG2 + c], sv, Dv * dysk);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kSB2 / 2; ++p) red_s[wv][p][lane] = rr[p];
    lds_barrier();
    {   // one output per thread: token m, value v (dB states 0-15 | dC states 0-15)
      const int m = tid >> 5, v = tid & 31, qn = v >> 4, sn = v & 15;
      const int t = tj + m;
      if (t < t1) {
        const float *rs = &red_s[0][0][0];
        const int off = (m >> 1) * 64 + 16 * ((m & 1) + 2 * qn) + sn;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kW2; ++w) sum += rs[w * (kSB2 / 2) * 64 + off];
        a.bc_part[((tb + t) * ncg + cg) * 32 + v] = sum;
      }
    }
    flush_dp_du(j);
  }
  a.dA_part[so] = dA;
  // the D gradient: the 16 staging threads of each channel add their columns in a fixed order
  __syncthreads();
  st_s[tid] = dDs;
  __syncthreads();
  if (tid < kCG2) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kSB2; ++q) s += st_s[q * kCG2 + tid];
    a.dD_part[((int64_t)b * a.nr + r) * a.D + cg * kCG2 + tid] = s;
  }
}

// dB | dC [T, 32] = sum over the channel groups of the scan's per-workgroup rows
__global__ __launch_bounds__(256) void bw_rowsum_kernel(const float *part, float *out, int64_t T,
                                                        int ncg) {
  // 4 consecutive values per thread (16-byte loads), each summed over the groups in order
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= T * 8) return;
  const int64_t tok = e >> 3;
  const int c = (int)(e & 7) * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int g = 0; g < ncg; ++g) {
    const float4 v = *(const float4 *)(part + (tok * ncg + g) * 32 + c);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *(float4 *)(out + tok * 32 + c) = s;
}

// ---------------------------------------------------------------- column sums
// part[blk][c] = sum of rows [blk * kColRows, +kColRows) of column c; then out[c] = sum_blk
// V4: 4 consecutive columns per thread (cols % 4 == 0). Rows are added in order either way;
// the unrolled loop lets the loads of 8 rows be in flight together.
template <bool V4>
__global__ __launch_bounds__(256) void bw_colsum_part_kernel(const float *in, int64_t rows,
                                                             int64_t cols, float *part) {
  const int64_t c = (blockIdx.x * 256ll + threadIdx.x) * (V4 ? 4 : 1);
  const int64_t blk = blockIdx.y;
  if (c >= cols) return;
  const int64_t r0 = blk * kColRows, r1 = min(rows, r0 + kColRows);
  if (V4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int64_t rr = r0; rr < r1; ++rr) {
      const float4 v = *(const float4 *)(in + rr * cols + c);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    *(float4 *)(part + blk * cols + c) = s;
  } else {
    float s = 0.f;
#pragma unroll 8
    for (int64_t rr = r0; rr < r1; ++rr) s += in[rr * cols + c];
    part[blk * cols + c] = s;
  }
}
__global__ __launch_bounds__(256) void bw_colsum_final_kernel(const float *part, int64_t nblk,
                                                              int64_t cols, float *out) {
  const int64_t c = blockIdx.x * 256ll + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int64_t k = 0; k < nblk; ++k) s += part[k * cols + c];
  out[c] = s;
}

// ---------------------------------------------------------------- RMSNorm backward
// one wave per token; slices [0, R) dt_low, [R, R+16) B, [R+16, R+32) C of xdbl
__global__ __launch_bounds__(256) void bw_norm_bwd_kernel(BwArgs a) {
  const int64_t tok = blockIdx.x * 4ll + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= a.T) return;
  const int W = a.R + 32;
  const float *v = a.xd + tok * W;
  float *dv = a.dxd + tok * W, *gc = a.gc + tok * W;
  auto slice = [&](int off, int len, const float *gamma, const float *dout) {
    float ss = 0.f, sg = 0.f;
    for (int j = lane; j < len; j += 64) {
      const float x = v[off + j];
      ss = __builtin_fmaf(x, x, ss);
      sg = __builtin_fmaf(gamma[j] * dout[j], x, sg);
    }
    ss = wave_sum(ss);
    sg = wave_sum(sg);
    const float rinv = 1.0f / sqrtf(ss / (float)len + a.eps);
    const float c = sg * rinv * rinv * rinv / (float)len;
    for (int j = lane; j < len; j += 64) {
      const float x = v[off + j];
      dv[off + j] = gamma[j] * dout[j] * rinv - x * c;
      gc[off + j] = dout[j] * x * rinv;
    }
  };
  slice(0, a.R, a.g_dt, a.ddtn + tok * a.R);
  slice(a.R, 16, a.g_B, a.dbc + tok * 32);
  slice(a.R + 16, 16, a.g_C, a.dbc + tok * 32 + 16);
}

// ---------------------------------------------------------------- conv + SiLU backward
// One thread per (sequence, strip of kStrip tokens, 4 channels). Walking t' over the strip
// (and K-1 tokens past it), it recomputes q(t') from a sliding window of x, forms
// dq = du SiLU'(q), and keeps the last K values of dq: dx[t] = sum_k w_k dq[t + K-1-k] is
// complete once t' = t + K-1. Partial sums of dq x(t - (K-1) + k) (d conv_w) and of dq
// (d conv_b) per strip go to conv_part [strips][D][5]; the strip at t = 0 also forms the
// carried conv state's gradient.
constexpr int kStrip = 64;
template <typename T, int K>
__global__ __launch_bounds__(256) void bw_conv_bwd_kernel(BwArgs a) {
  const int nq = a.D / 4;
  const int nstrip = (a.L + kStrip - 1) / kStrip;
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= (int64_t)a.B * nstrip * nq) return;
  const int i0 = (int)(e % nq) * 4;
  const int strip = (int)((e / nq) % nstrip), b = (int)(e / ((int64_t)nq * nstrip));
  const int t0 = strip * kStrip, t1 = min(a.L, t0 + kStrip);
  const int64_t tb = (int64_t)b * a.L;
  float w[4][K], bias[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    bias[c] = a.conv_b ? io<T>::ld((const T *)a.conv_b + i0 + c) : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) w[c][k] = io<T>::ld((const T *)a.conv_w + (i0 + c) * K + k);
  }
  float xw[K][4];                 // xw[k] = x(t' - (K-1) + k)
#pragma unroll
  for (int k = 0; k < K - 1; ++k) conv_in4<T>(a, b, t0 - (K - 1) + k, i0, xw[k]);
  float dqr[K][4];                // dqr[K-1-j] = dq(t' - j)
  float first[K][4];              // dq(0 .. K-2) of the strip at t = 0
  float pw[K][4], pb[4];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) dqr[k][c] = pw[k][c] = first[k][c] = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) pb[c] = 0.f;
  for (int tp = t0; tp < t1 + K - 1; ++tp) {
    float dq[4] = {0.f, 0.f, 0.f, 0.f};
    if (tp < a.L) {
      conv_in4<T>(a, b, tp, i0, xw[K - 1]);
      float du[4];
      v4io<float>::ld(a.du + (tb + tp) * a.D + i0, du);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float q = bias[c];
#pragma unroll
        for (int k = 0; k < K; ++k) q = __builtin_fmaf(w[c][k], xw[k][c], q);
        dq[c] = du[c] * dsilu_f(q);
      }
      if (tp < t1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pb[c] += dq[c];
#pragma unroll
          for (int k = 0; k < K; ++k) pw[k][c] = __builtin_fmaf(dq[c], xw[k][c], pw[k][c]);
        }
      }
      if (tp < K - 1) {
#pragma unroll
        for (int k = 0; k < K - 1; ++k)
          if (tp == k)
#pragma unroll
            for (int c = 0; c < 4; ++c) first[k][c] = dq[c];
      }
    }
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        dqr[k][c] = dqr[k + 1][c];
        xw[k][c] = xw[k + 1][c];
      }
#pragma unroll
    for (int c = 0; c < 4; ++c) dqr[K - 1][c] = dq[c];
    const int t = tp - (K - 1);
    if (t >= t0) {
      float dx[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) v = __builtin_fmaf(w[c][k], dqr[K - 1 - k][c], v);
        dx[c] = v;
      }
      v4io<T>::st((T *)a.dxz + (tb + t) * 2 * a.D + i0, dx);
    }
  }
  float *cp = a.conv_part + (((int64_t)b * nstrip + strip) * a.D + i0) * 5;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int k = 0; k < K; ++k) cp[c * 5 + k] = pw[k][c];
#pragma unroll
    for (int k = K; k < 4; ++k) cp[c * 5 + k] = 0.f;
    cp[c * 5 + 4] = pb[c];
  }
  if (strip == 0 && a.d_conv_state) {
    // position s in [-(K-1), 0): sum over k of w_k dq(s + K-1-k), dq known for 0 <= . < L
#pragma unroll
    for (int sidx = 0; sidx < K - 1; ++sidx) {
      const int sp = sidx - (K - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int q = sp + K - 1 - k;
          if (q >= 0 && q < K - 1 && q < a.L) d = __builtin_fmaf(w[c][k], first[q][c], d);
        }
        a.d_conv_state[((int64_t)b * a.D + i0 + c) * (K - 1) + sidx] = d;
      }
    }
  }
}
// column sums of conv_part, [D][5] in conv_sum -> d conv_w [D, K], d conv_b [D]
__global__ __launch_bounds__(256) void bw_conv_scatter_kernel(BwArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.D) return;
  for (int k = 0; k < a.K; ++k) a.d_conv_w[i * a.K + k] = a.conv_sum[i * 5 + k];
  if (a.d_conv_b) a.d_conv_b[i] = a.conv_sum[i * 5 + 4];
}

// ---------------------------------------------------------------- fp32 GEMM
// C[m scm + n scn] (+)= sum_k A(m, k) B(k, n), A(m, k) = A[m sam + k sak],
// B(k, n) = B[k sbk + n sbn]. BM x BN tiles, 4 waves of (BM/2) x (BN/2) (blocks of
// v_mfma_f32_16x16x4_f32), K in chunks of 16 through LDS; rows padded to a stride of 16 mod 64
// floats so that the 4 k-rows of a fragment read fall in distinct bank groups. The next chunk's
// elements are loaded into registers while the current chunk is multiplied.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args g) {
  constexpr int PA = BM + 16, PB = BN + 16;
  constexpr int NA = BM * 16 / 256, NB = BN * 16 / 256;   // elements per thread per chunk
  constexpr int XB = BM / 32, YB = BN / 32;               // 16 x 16 blocks per wave
  __shared__ float as[16 * PA], bs[16 * PB];
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int l16 = lane & 15, lk = lane >> 4;
  // split-K: this workgroup's K range (chunks of 16 per split)
  const int kc = ((g.K + g.split - 1) / g.split + 15) / 16 * 16;
  const int kbeg = blockIdx.z * kc, kend = min(g.K, kbeg + kc);
  float ra[NA], rb[NB];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int e = tid + 256 * j;
      const int mm = g.sak == 1 ? e >> 4 : e % BM, kk = g.sak == 1 ? e & 15 : e / BM;
      const int m = m0 + mm, k = k0 + kk;
      ra[j] = (m < g.M && k < kend) ? g.A[(int64_t)m * g.sam + (int64_t)k * g.sak] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = tid + 256 * j;
      const int nn = g.sbn == 1 ? e % BN : e >> 4, kk = g.sbn == 1 ? e / BN : e & 15;
      const int n = n0 + nn, k = k0 + kk;
      rb[j] = (n < g.N && k < kend) ? g.B[(int64_t)k * g.sbk + (int64_t)n * g.sbn] : 0.f;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int e = tid + 256 * j;
      if (g.sak == 1) as[(e & 15) * PA + (e >> 4)] = ra[j];
      else as[(e / BM) * PA + e % BM] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = tid + 256 * j;
      if (g.sbn == 1) bs[(e / BN) * PB + e % BN] = rb[j];
      else bs[(e & 15) * PB + (e >> 4)] = rb[j];
    }
  };
  f32x4 acc[XB][YB];
#pragma unroll
  for (int x = 0; x < XB; ++x)
#pragma unroll
    for (int y = 0; y < YB; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    stash();
    __syncthreads();
    if (k0 + 16 < kend) load(k0 + 16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kr = ks * 4 + lk;
      float fa[XB], fb[YB];
#pragma unroll
      for (int x = 0; x < XB; ++x) fa[x] = as[kr * PA + wm * (BM / 2) + x * 16 + l16];
#pragma unroll
      for (int y = 0; y < YB; ++y) fb[y] = bs[kr * PB + wn * (BN / 2) + y * 16 + l16];
      // lane (l16, lk) of block (x, y) ends with C[m = 16 x + 4 lk + q][n = 16 y + l16]
#pragma unroll
      for (int x = 0; x < XB; ++x)
#pragma unroll
        for (int y = 0; y < YB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < XB; ++x)
#pragma unroll
    for (int y = 0; y < YB; ++y)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * (BM / 2) + x * 16 + lk * 4 + q;
        const int n = n0 + wn * (BN / 2) + y * 16 + l16;
        if (m < g.M && n < g.N) {
          if (g.split > 1) {
            g.part[((int64_t)blockIdx.z * g.M + m) * g.N + n] = acc[x][y][q];
          } else {
            float *c = g.C + (int64_t)m * g.scm + (int64_t)n * g.scn;
            *c = g.accumulate ? *c + acc[x][y][q] : acc[x][y][q];
          }
        }
      }
}

// split-K: C[m scm + n scn] (+)= sum over splits of part[split][m][n], in split order
__global__ __launch_bounds__(256) void gemm_f32_splitk_sum_kernel(GemmF32Args g) {
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= (int64_t)g.M * g.N) return;
  const int64_t m = e / g.N, n = e % g.N;
  float v = 0.f;
  for (int z = 0; z < g.split; ++z) v += g.part[(int64_t)z * g.M * g.N + e];
  float *c = g.C + m * g.scm + n * g.scn;
  *c = g.accumulate ? *c + v : v;
}

inline unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 65536 ? b : 65536);
}

}  // namespace

int gemm_f32_split(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + 127) / 128) * (N <= 512 ? (N + 63) / 64 : (N + 127) / 128);
  int split = 1;
  while (split < kMaxSplit && tiles * split < 1024 && K / (split * 2) >= 2048) split *= 2;
  return split;
}

hipError_t launch_gemm_f32(const GemmF32Args &g0, hipStream_t s) {
  if (g0.M <= 0 || g0.N <= 0) return hipSuccess;
  GemmF32Args g = g0;
  g.split = g.part ? gemm_f32_split(g.M, g.N, g.K) : 1;
  if (g.N <= 512)
    hipLaunchKernelGGL((gemm_f32_kernel<128, 64>),
                       dim3((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 127) / 128), (unsigned)g.split),
                       dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<128, 128>),
                       dim3((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128), (unsigned)g.split),
                       dim3(256), 0, s, g);
  if (g.split > 1)
    hipLaunchKernelGGL(gemm_f32_splitk_sum_kernel, dim3((unsigned)(((int64_t)g.M * g.N + 255) / 256)),
                       dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_colsum(const float *in, int64_t rows, int64_t cols, float *part, float *out,
                         hipStream_t s) {
  const int64_t nblk = (rows + kColRows - 1) / kColRows;
  if (cols % 4 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)part & 15) == 0)
    hipLaunchKernelGGL(bw_colsum_part_kernel<true>,
                       dim3((unsigned)((cols / 4 + 255) / 256), (unsigned)nblk), dim3(256), 0, s,
                       in, rows, cols, part);
  else
    hipLaunchKernelGGL(bw_colsum_part_kernel<false>,
                       dim3((unsigned)((cols + 255) / 256), (unsigned)nblk), dim3(256), 0, s, in,
                       rows, cols, part);
  hipLaunchKernelGGL(bw_colsum_final_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, s,
                     part, nblk, cols, out);
  return hipGetLastError();
}

int bw_ranges(int L) { return (L + kRT - 1) / kRT; }
int bw_conv_strips(int L) { return (L + kStrip - 1) / kStrip; }
int64_t bw_colsum_blocks(int64_t rows) { return (rows + kColRows - 1) / kColRows; }

template <typename T>
hipError_t bw_dispatch(const BwArgs &a, int stage, hipStream_t s) {
  switch (stage) {
    case 0: {
      const dim3 grid((unsigned)(a.B * ((a.L + kUStrip - 1) / kUStrip)), (unsigned)((a.D + 1023) / 1024));
      if (a.K == 2) hipLaunchKernelGGL((bw_conv_u_kernel<T, 2>), grid, dim3(256), 0, s, a);
      else if (a.K == 3) hipLaunchKernelGGL((bw_conv_u_kernel<T, 3>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((bw_conv_u_kernel<T, 4>), grid, dim3(256), 0, s, a);
      break;
    }
    case 2: {
      const dim3 rgrid((unsigned)(a.B * a.nr * (a.D / kCG)));
      if (a.zoh) hipLaunchKernelGGL((bw_range_transfer_kernel<T, true>), rgrid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((bw_range_transfer_kernel<T, false>), rgrid, dim3(256), 0, s, a);
      const int64_t nc = (int64_t)a.B * a.D * 16;
      hipLaunchKernelGGL(bw_range_carry_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, a);
      const unsigned grid = (unsigned)(a.B * a.nr * (a.D / kCG2));
      if (a.zoh) hipLaunchKernelGGL((bw_scan_kernel<T, true>), dim3(grid), dim3(kST2), 0, s, a);
      else hipLaunchKernelGGL((bw_scan_kernel<T, false>), dim3(grid), dim3(kST2), 0, s, a);
      hipLaunchKernelGGL(bw_rowsum_kernel, dim3((unsigned)((a.T * 8 + 255) / 256)), dim3(256), 0, s,
                         a.bc_part, a.dbc, a.T, a.D / kCG2);
      break;
    }
    case 3:
      hipLaunchKernelGGL(bw_norm_bwd_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
      break;
    case 5: {
      const int64_t nth = (int64_t)a.B * ((a.L + kStrip - 1) / kStrip) * (a.D / 4);
      const dim3 grid((unsigned)((nth + 255) / 256));
      if (a.K == 2) hipLaunchKernelGGL((bw_conv_bwd_kernel<T, 2>), grid, dim3(256), 0, s, a);
      else if (a.K == 3) hipLaunchKernelGGL((bw_conv_bwd_kernel<T, 3>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((bw_conv_bwd_kernel<T, 4>), grid, dim3(256), 0, s, a);
      break;
    }
    case 7:
      hipLaunchKernelGGL(bw_conv_scatter_kernel, dim3((unsigned)((a.D + 255) / 256)), dim3(256), 0, s, a);
      break;
    case 6: {  // weights to fp32 (bf16 I/O)
      const int W = a.R + 32;
      hipLaunchKernelGGL(to_f32_kernel<T>, dim3(grid_for((int64_t)W * a.D)), dim3(256), 0, s,
                         (const T *)a.x_proj_w, a.wx32, (int64_t)W * a.D);
      hipLaunchKernelGGL(to_f32_kernel<T>, dim3(grid_for((int64_t)a.D * a.R)), dim3(256), 0, s,
                         (const T *)a.dt_proj_w, a.wdt32, (int64_t)a.D * a.R);
      break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_backward_stage(mm_dtype dt, const BwArgs &a, int stage, hipStream_t s) {
  return dt == MM_F32 ? bw_dispatch<float>(a, stage, s) : bw_dispatch<bf16_t>(a, stage, s);
}

}  // namespace mm
