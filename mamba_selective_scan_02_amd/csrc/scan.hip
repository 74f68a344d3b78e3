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
  float Av[kN], A2[kN], iA[kN], h[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    Av[n] = a.A[(int64_t)i * kN + n];
    A2[n] = Av[n] * kLog2e;
    iA[n] = 1.0f / Av[n];
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
        const float em1 = expm1_f(dt * Av[n]);
        const float dA = em1 + 1.0f;
        h[n] = __builtin_fmaf(dA, h[n], em1 * iA[n] * Bt[n] * u);
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

// ---------------------------------------------------------------------------------------
// Time-parallel scan for long sequences (few sequences x channels to fill 256 CUs).
//
// A workgroup owns kCh = 32 channels of one sequence and walks the sequence in blocks of
// kW * kS = 128 tokens. Each of its kW = 8 waves takes one kS = 16-token segment of a block.
// Lane l works on channel l/2 and on the 8 states 8*(l%2) .. 8*(l%2)+7 of it.
//  1. Local pass: the segment is scanned from h = 0, keeping exp(dt*A) of every
//     (token, state) in VGPRs (one exp per element, as in the sequential recurrence).
//  2. The segment's transfer (P, S) -- h_out = P * h_in + S with P = exp(A * sum dt) and S the
//     local end state -- goes to LDS; each wave composes the transfers of the segments before
//     it onto the block's carry-in, with the page's associative scan operator
//     ("Parallel training via the parallel scan": (a, b) then (c, d) gives (ac, ad + b) for
//     the map h -> a h + b), and every wave also composes all 8 to get the next carry-in.
//  3. Replay: the segment is run again from its true h_in with the stored exp(dt*A), and
//     y_t = C_t . h_t is formed; the two half-sums of a channel meet by a DPP lane swap.
// x, z, dt of the block are staged through LDS with 16-byte loads; so are B, C (shared by all
// channels of a token). The conv window needs 3 tokens before the block (carried state or 0
// before token 0).
constexpr int kCh = 32, kW = 8, kS = 16, kG = 8, kBlk = kW * kS;

template <typename T, bool ZOH, int K>
__global__ __launch_bounds__(kW * 64) void scan_chunked_kernel(ScanArgs a) {
  typedef typename Delta<T>::type DT;
  constexpr int kHalo = 3;  // rows before the block kept for the conv window (K - 1 <= 3)
  __shared__ __attribute__((aligned(16))) float bc_s[kBlk][2 * kN];
  __shared__ __attribute__((aligned(16))) float agg_s[kW][64][2 * kG];
  __shared__ __attribute__((aligned(16))) T x_s[kBlk + kHalo][kCh];
  __shared__ __attribute__((aligned(16))) T z_s[kBlk][kCh];
  __shared__ __attribute__((aligned(16))) DT d_s[kBlk][kCh];
  // per-token u and dt*u (ZOH: u) of this block, written and read by the same wave
  __shared__ float u_s[kBlk][kCh];
  __shared__ float du_s[kBlk][kCh];

  const int groups = a.D / kCh;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = gid / groups;
  const int ch0 = (gid % groups) * kCh;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int c = lane >> 1, p = lane & 1;
  const int ch = ch0 + c;

  float A2[kG], Av[kG], iA[kG], carry[kG];
#pragma unroll
  for (int j = 0; j < kG; ++j) {
    Av[j] = a.A[(int64_t)ch * kN + kG * p + j];
    A2[j] = Av[j] * kLog2e;
    iA[j] = 1.0f / Av[j];
    carry[j] = (a.state_valid && a.state) ? a.state[((int64_t)b * a.D + ch) * kN + kG * p + j] : 0.f;
  }
  float wc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wc[k] = io<T>::cvt(((const T *)a.conv_w)[(int64_t)ch * K + k]);
  const float cb = a.conv_b ? io<T>::cvt(((const T *)a.conv_b)[ch]) : 0.0f;
  const float Dv = a.Dskip[ch];

  const int64_t row = 2LL * a.D;
  const T *xzb = (const T *)a.xz + (int64_t)b * a.L * row;
  const DT *db = (const DT *)a.delta + (int64_t)b * a.L * a.D;
  const float *bcb = a.bc + (int64_t)b * a.L * 2 * kN;
  T *yb = (T *)a.y + (int64_t)b * a.L * a.D;
  const int nblocks = (a.L + kBlk - 1) / kBlk;

  for (int blk = 0; blk < nblocks; ++blk) {
    const int T0 = blk * kBlk;
    __syncthreads();  // previous block's readers are done with the LDS tiles
    // ---- stage B|C rows (128 B each), 4 threads per token
    {
      const int tk = tid >> 2, q = tid & 3;
      float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
      if (T0 + tk < a.L) {
        const float4 *src = (const float4 *)(bcb + (int64_t)(T0 + tk) * 2 * kN + 8 * q);
        v0 = src[0];
        v1 = src[1];
      }
      *(float4 *)&bc_s[tk][8 * q] = v0;
      *(float4 *)&bc_s[tk][8 * q + 4] = v1;
    }
    // ---- stage x (with halo), z and dt rows: 32 channels = 64 B per row = 4 x 16 B
    constexpr int xper = 16 / sizeof(T);   // elements per 16-byte chunk
    constexpr int xcpr = kCh / xper;       // chunks per 32-channel row
    for (int e = tid; e < (kBlk + kHalo) * xcpr; e += kW * 64) {
      const int r = e / xcpr, q = e % xcpr;
      const int t = T0 - kHalo + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t >= 0 && t < a.L) {
        v = *(const uint4 *)(xzb + (int64_t)t * row + ch0 + q * xper);
      } else if (t < 0 && a.conv_valid && a.conv_state && t >= -(K - 1)) {
        // carried conv state, oldest first: row t = -(K-1)+j holds conv_state[b, ch, j]
        T tmp[xper];
#pragma unroll
        for (int e2 = 0; e2 < xper; ++e2) {
          const int chh = ch0 + q * xper + e2;
          tmp[e2] = ((const T *)a.conv_state)[((int64_t)b * a.D + chh) * (K - 1) + (K - 1) + t];
        }
        v = *(const uint4 *)tmp;
      }
      *(uint4 *)&x_s[r][q * xper] = v;
    }
    for (int e = tid; e < kBlk * xcpr; e += kW * 64) {
      const int r = e / xcpr, q = e % xcpr;
      const int t = T0 + r;
      uint4 vz = make_uint4(0, 0, 0, 0);
      if (t < a.L) vz = *(const uint4 *)(xzb + (int64_t)t * row + a.D + ch0 + q * xper);
      *(uint4 *)&z_s[r][q * xper] = vz;
    }
    for (int e = tid; e < kBlk * (kCh * (int)sizeof(DT) / 16); e += kW * 64) {
      constexpr int per = 16 / sizeof(DT);           // elements per 16-byte chunk
      constexpr int cpr = kCh / per;                 // chunks per row
      const int r = e / cpr, q = e % cpr;
      const int t = T0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < a.L) v = *(const uint4 *)(db + (int64_t)t * a.D + ch0 + q * per);
      *(uint4 *)&d_s[r][q * per] = v;
    }
    __syncthreads();

    // ---- 1. local pass over this wave's segment
    const int tb0 = wv * kS;
    float win[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) win[j] = io<T>::cvt(x_s[tb0 + kHalo - (K - 1) + j][c]);
    float dA[kS][kG];
    float hl[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) hl[j] = 0.f;
    float sumdt = 0.f;
#pragma unroll
    for (int t = 0; t < kS; ++t) {
      const int tb = tb0 + t;
      const float x = io<T>::cvt(x_s[tb + kHalo][c]);
      float acc = cb;
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc = __builtin_fmaf(wc[j], win[j], acc);
      acc = __builtin_fmaf(wc[K - 1], x, acc);
#pragma unroll
      for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
      win[K - 2] = x;
      const float u = silu_f(acc);
      const float dt = (float)d_s[tb][c];
      sumdt += dt;
      u_s[tb][c] = u;
      const float4 B0 = *(const float4 *)&bc_s[tb][kG * p];
      const float4 B1 = *(const float4 *)&bc_s[tb][kG * p + 4];
      const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
      if (ZOH) {
        du_s[tb][c] = u;
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          const float em1 = expm1_f(dt * Av[j]);
          dA[t][j] = em1;  // ZOH keeps expm1(dt A); exp(dt A) = 1 + it
          hl[j] = __builtin_fmaf(em1 + 1.0f, hl[j], em1 * iA[j] * Bv[j] * u);
        }
      } else {
        const float du = dt * u;
        du_s[tb][c] = du;
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          dA[t][j] = exp2_hw(dt * A2[j]);
          hl[j] = __builtin_fmaf(dA[t][j], hl[j], du * Bv[j]);
        }
      }
    }
    // ---- 2. publish this segment's transfer h -> P h + S
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      agg_s[wv][lane][j] = exp2_hw(A2[j] * sumdt);
      agg_s[wv][lane][kG + j] = hl[j];
    }
    __syncthreads();
    // ---- compose: h_in of this segment, and the carry into the next block
    float hin[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) hin[j] = carry[j];
    for (int w2 = 0; w2 < kW; ++w2) {
      if (w2 == wv) {
#pragma unroll
        for (int j = 0; j < kG; ++j) hin[j] = carry[j];
      }
      const float4 *ag = (const float4 *)&agg_s[w2][lane][0];
      const float4 P0 = ag[0], P1 = ag[1], S0 = ag[2], S1 = ag[3];
      const float Pv[kG] = {P0.x, P0.y, P0.z, P0.w, P1.x, P1.y, P1.z, P1.w};
      const float Sv[kG] = {S0.x, S0.y, S0.z, S0.w, S1.x, S1.y, S1.z, S1.w};
#pragma unroll
      for (int j = 0; j < kG; ++j) carry[j] = __builtin_fmaf(Pv[j], carry[j], Sv[j]);
    }
    // ---- 3. replay from the true h_in; y from the two half-sums of the channel
    float h[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) h[j] = hin[j];
#pragma unroll
    for (int t = 0; t < kS; t += 2) {
      float ys[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tb = tb0 + t + e;
        const float4 B0 = *(const float4 *)&bc_s[tb][kG * p];
        const float4 B1 = *(const float4 *)&bc_s[tb][kG * p + 4];
        const float4 C0 = *(const float4 *)&bc_s[tb][kN + kG * p];
        const float4 C1 = *(const float4 *)&bc_s[tb][kN + kG * p + 4];
        const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
        const float Cv[kG] = {C0.x, C0.y, C0.z, C0.w, C1.x, C1.y, C1.z, C1.w};
        const float du = du_s[tb][c];
        float yy = 0.f;
#pragma unroll
        for (int j = 0; j < kG; ++j) {
          if (ZOH) {
            const float em1 = dA[t + e][j];
            h[j] = __builtin_fmaf(em1 + 1.0f, h[j], em1 * iA[j] * Bv[j] * du);
          } else {
            h[j] = __builtin_fmaf(dA[t + e][j], h[j], du * Bv[j]);
          }
          yy = __builtin_fmaf(Cv[j], h[j], yy);
        }
        ys[e] = yy;
      }
      // lane p keeps token t+p: its own half-sum plus the partner lane's half-sum of it
      const float keep = p ? ys[1] : ys[0];
      const float send = p ? ys[0] : ys[1];
      const float other = __builtin_bit_cast(
          float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
      const int tb = tb0 + t + p;
      const float u = u_s[tb][c];
      const float z = io<T>::cvt(z_s[tb][c]);
      const float yv = __builtin_fmaf(Dv, u, keep + other) * silu_f(z);
      if (T0 + tb < a.L) io<T>::st(yb + (int64_t)(T0 + tb) * a.D + ch, yv);
    }
  }
  if (a.state && wv == 0) {
#pragma unroll
    for (int j = 0; j < kG; ++j) a.state[((int64_t)b * a.D + ch) * kN + kG * p + j] = carry[j];
  }
}

template <typename T, int K>
hipError_t dispatch_chunked_k(const ScanArgs &a, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)a.B * (a.D / kCh));
  if (a.zoh)
    hipLaunchKernelGGL((scan_chunked_kernel<T, true, K>), dim3(blocks), dim3(kW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((scan_chunked_kernel<T, false, K>), dim3(blocks), dim3(kW * 64), 0, s, a);
  return hipGetLastError();
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

// The sequential kernel has one wave per 64 (sequence, channel) pairs; when that leaves the
// chip underfilled (fewer than 2048 waves) and the sequence is long, the time-parallel kernel
// runs instead.
bool use_chunked(const ScanArgs &a) {
  if (a.force == 1) return false;
  if (a.force == 2) return a.D % kCh == 0;
  const int64_t waves = (int64_t)a.B * a.D / 64;
  return a.L > kBlk && waves < 2048 && a.D % kCh == 0;
}

template <typename T>
hipError_t dispatch(const ScanArgs &a, hipStream_t s) {
  const bool ch = use_chunked(a);
  switch (a.K) {
    case 2: return ch ? dispatch_chunked_k<T, 2>(a, s) : dispatch_k<T, 2>(a, s);
    case 3: return ch ? dispatch_chunked_k<T, 3>(a, s) : dispatch_k<T, 3>(a, s);
    case 4: return ch ? dispatch_chunked_k<T, 4>(a, s) : dispatch_k<T, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan(mm_dtype dt, const ScanArgs &a, hipStream_t s) {
  if (a.N != kN) return hipErrorInvalidValue;
  return dt == MM_BF16 ? dispatch<bf16_t>(a, s) : dispatch<float>(a, s);
}

}  // namespace mm
