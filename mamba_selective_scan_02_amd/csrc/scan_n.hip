// Selective scan + D feed-through + SiLU(z) gate for state sizes other than 16 (d_state 8, 32,
// 64: the state-size sweep around the N = 16 of the Jamba configuration).
//
// Same recurrence as scan.hip (Jamba analysis page, "The Mamba Layer": ZOH equation, discrete
// recurrence, the D u feed-through of the continuous SSM; Mamba-1 gate), cut into ranges of
// kGR tokens and composed with the page's associative operator ("Parallel training via the
// parallel scan": h -> a h + b composes as (a, b) then (c, d) = (ac, ad + b)):
//   scanN_transfer_kernel  per (range, channel, state): the range's transfer h -> P h + S from
//                          zero (P = prod exp(dt A), S = the local end state)
//   scanN_carry_kernel     per (sequence, channel, state), sequential over ranges: each range's
//                          true start state (written over S) and the final state
//   scanN_replay_kernel    per range: the recurrence from the true start state, y_t = C_t . h_t
//                          summed over the N state lanes (DPP mirrors within 8 / 16 lanes, lane
//                          swaps across 16-lane rows), y = (y + D u) SiLU(z)
// Lanes are (channel, group of S consecutive states; S = 1 for N = 8, N / 16 otherwise): N / S
// lanes per channel (8 for N = 8, 16 otherwise), so a workgroup of 256 threads covers 256 S / N
// channels and the sum over states is one 8- or 16-lane DPP reduction per token, shared by S
// states. (Two states per lane for N = 8 measured slower: 64 channels per workgroup raise the
// staged prefetch to 26 registers per thread.) Each
// kGS-token sub-block's inputs are staged in LDS by coalesced loads issued one sub-block ahead.
// u comes from the conv kernel's output (fp32, or bf16 high + low parts: ~2^-17 relative).
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

constexpr int kGR = 512;   // tokens per range
constexpr int kGS = 32;    // tokens per staged sub-block

// Prefetched elements travel as raw bits and are decoded when they are staged: decoding a
// 16-bit value where it is loaded would make the wave wait for the load one sub-block early.
// dt: fp32; u: fp32, or bf16 high | low parts; z: the I/O type.
template <typename T> struct Raw;
template <> struct Raw<float> {
  static __device__ __forceinline__ uint32_t dt(const ScanArgs &a, int64_t e) {
    return __float_as_uint(((const float *)a.delta)[e]);
  }
  static __device__ __forceinline__ uint32_t u(const ScanArgs &a, int64_t e) {
    return __float_as_uint(((const float *)a.u)[e]);
  }
  static __device__ __forceinline__ uint32_t z(const ScanArgs &a, int64_t e) {
    return __float_as_uint(((const float *)a.xz)[e]);
  }
  static __device__ __forceinline__ float dt_f(uint32_t v) { return __uint_as_float(v); }
  static __device__ __forceinline__ float u_f(uint32_t v) { return __uint_as_float(v); }
  static __device__ __forceinline__ float z_f(uint32_t v) { return __uint_as_float(v); }
};
template <> struct Raw<bf16_t> {
  static __device__ __forceinline__ uint32_t dt(const ScanArgs &a, int64_t e) {
    return __float_as_uint(((const float *)a.delta)[e]);
  }
  static __device__ __forceinline__ uint32_t u(const ScanArgs &a, int64_t e) {
    return (uint32_t)((const bf16_t *)a.u)[e] | ((uint32_t)((const bf16_t *)a.u_lo)[e] << 16);
  }
  static __device__ __forceinline__ uint32_t z(const ScanArgs &a, int64_t e) {
    return ((const bf16_t *)a.xz)[e];
  }
  static __device__ __forceinline__ float dt_f(uint32_t v) { return __uint_as_float(v); }
  static __device__ __forceinline__ float u_f(uint32_t v) {
    return bf2f((bf16_t)(v & 0xFFFFu)) + bf2f((bf16_t)(v >> 16));
  }
  static __device__ __forceinline__ float z_f(uint32_t v) { return bf2f((bf16_t)v); }
};

// sum over the G lanes of a channel (G = 4, 8 or 16, groups aligned to G lanes); every lane
// of the group receives it. All source lanes lie inside the row (bound_ctrl changes no value
// and lets each move fold into its add).
template <int G>
__device__ __forceinline__ float sum_group(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // ^1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // ^2
  if (G >= 8)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // 7-i
  if (G >= 16)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // 15-i
  return v;
}
template <int N> constexpr int states_per_lane() { return N >= 16 ? N / 16 : 1; }

// S consecutive floats of a staged row (8- or 16-byte LDS reads for S = 2, 4)
template <int S>
__device__ __forceinline__ void lds_vec(const float *p, float v[S]) {
  if (S == 4) {
    const float4 x = *(const float4 *)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else if (S == 2) {
    const float2 x = *(const float2 *)p;
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = p[0];
  }
}

template <typename T, int N, bool ZOH>
__global__ __launch_bounds__(256) void scanN_transfer_kernel(ScanArgs a, int nr) {
  constexpr int S = states_per_lane<N>(), G = N / S;
  constexpr int CPW = 256 / G;             // channels per workgroup
  constexpr int F = kGS * CPW;             // floats of a staged [kGS][CPW] array
  constexpr int ST = 2 * F + kGS * N;      // dt | u | B
  constexpr int NQ = (ST + 255) / 256;
  __shared__ __attribute__((aligned(16))) float st_s[NQ * 256];
  const int ncg = a.D / CPW;
  const int cg = blockIdx.x % ncg;
  const int r = (blockIdx.x / ncg) % nr;
  const int b = blockIdx.x / (ncg * nr);
  const int tid = threadIdx.x, j = tid % G, c = tid / G, i = cg * CPW + c;
  const int n0 = j * S;                    // this lane's states n0 .. n0 + S - 1
  const int t0 = r * kGR, t1 = min(a.L, t0 + kGR);
  const int nsb = (t1 - t0 + kGS - 1) / kGS;
  const int64_t tb = (int64_t)b * a.L;
  float An[S], A2[S], iA[S], P[S], Sv[S];
#pragma unroll
  for (int q = 0; q < S; ++q) {
    An[q] = a.A[(int64_t)i * N + n0 + q];
    A2[q] = An[q] * kLog2e;
    iA[q] = 1.0f / An[q];
    P[q] = 1.f;
    Sv[q] = 0.f;
  }
  static_assert(F % 256 == 0, "each prefetch slot holds one kind of element");
  uint32_t pf[NQ];   // slot q < F/256: dt; < 2F/256: u; then B (raw bits, see Raw)
  auto fetch = [&](int jb) {
    const int tj = t0 + jb * kGS;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + 256 * q;
      uint32_t v = 0;
      if (e < 2 * F) {
        const int off = e % F, k = off / CPW, ch = off % CPW;
        const int64_t x = (tb + tj + k) * a.D + cg * CPW + ch;
        if (tj + k < t1) v = q < F / 256 ? Raw<T>::dt(a, x) : Raw<T>::u(a, x);
      } else if (e < ST) {
        const int off = e - 2 * F, k = off / N, nn = off % N;
        if (tj + k < t1) v = __float_as_uint(a.bc[(tb + tj + k) * 2 * N + nn]);
      }
      pf[q] = v;
    }
  };
  const float *s_dt = st_s, *s_u = st_s + F, *s_b = st_s + 2 * F;
  fetch(0);
  for (int jb = 0; jb < nsb; ++jb) {
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      st_s[tid + 256 * q] = q < F / 256 ? Raw<T>::dt_f(pf[q])
                            : q < 2 * F / 256 ? Raw<T>::u_f(pf[q]) : __uint_as_float(pf[q]);
    lds_barrier();
    if (jb + 1 < nsb) fetch(jb + 1);
    const int tj = t0 + jb * kGS;
#pragma unroll 4
    for (int k = 0; k < kGS; ++k) {
      if (tj + k < t1) {
        const float dtv = s_dt[k * CPW + c], uv = s_u[k * CPW + c];
        float Bv[S];
        lds_vec<S>(s_b + k * N + n0, Bv);
#pragma unroll
        for (int q = 0; q < S; ++q) {
          const float av = exp2_hw(dtv * A2[q]);
          const float bb = (ZOH ? expm1_f(dtv * An[q]) * iA[q] : dtv) * Bv[q];
          Sv[q] = __builtin_fmaf(av, Sv[q], bb * uv);
          P[q] *= av;
        }
      }
    }
  }
  const int64_t o = (((int64_t)b * nr + r) * a.D + i) * N + n0;
#pragma unroll
  for (int q = 0; q < S; ++q) {
    a.gP[o + q] = P[q];
    a.gS[o + q] = Sv[q];
  }
}

template <int N>
__global__ __launch_bounds__(256) void scanN_carry_kernel(ScanArgs a, int nr) {
  const int64_t e = blockIdx.x * 256ll + threadIdx.x;
  if (e >= (int64_t)a.B * a.D * N) return;
  const int64_t b = e / ((int64_t)a.D * N), in = e % ((int64_t)a.D * N);
  float h = (a.state_valid && a.state) ? a.state[e] : 0.f;
  for (int r = 0; r < nr; ++r) {
    const int64_t o = (b * nr + r) * a.D * N + in;
    const float s = a.gS[o];
    a.gS[o] = h;
    h = __builtin_fmaf(a.gP[o], h, s);
  }
  if (a.state) a.state[e] = h;
}

template <typename T, int N, bool ZOH>
__global__ __launch_bounds__(256) void scanN_replay_kernel(ScanArgs a, int nr) {
  constexpr int S = states_per_lane<N>(), G = N / S;
  constexpr int CPW = 256 / G;
  constexpr int F = kGS * CPW;
  constexpr int ST = 3 * F + kGS * 2 * N;  // dt | u | z | B|C
  constexpr int NQ = (ST + 255) / 256;
  __shared__ __attribute__((aligned(16))) float st_s[NQ * 256];
  const int ncg = a.D / CPW;
  const int cg = blockIdx.x % ncg;
  const int r = (blockIdx.x / ncg) % nr;
  const int b = blockIdx.x / (ncg * nr);
  const int tid = threadIdx.x, j = tid % G, c = tid / G, i = cg * CPW + c;
  const int n0 = j * S;
  const int t0 = r * kGR, t1 = min(a.L, t0 + kGR);
  const int nsb = (t1 - t0 + kGS - 1) / kGS;
  const int64_t tb = (int64_t)b * a.L;
  float An[S], A2[S], iA[S], h[S];
  const int64_t so = (((int64_t)b * nr + r) * a.D + i) * N + n0;
#pragma unroll
  for (int q = 0; q < S; ++q) {
    An[q] = a.A[(int64_t)i * N + n0 + q];
    A2[q] = An[q] * kLog2e;
    iA[q] = 1.0f / An[q];
    h[q] = a.gS[so + q];
  }
  const float Dv = a.Dskip[i];
  static_assert(F % 256 == 0, "each prefetch slot holds one kind of element");
  uint32_t pf[NQ];   // slot q < F/256: dt; < 2F/256: u; < 3F/256: z; then B|C (raw bits)
  auto fetch = [&](int jb) {
    const int tj = t0 + jb * kGS;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = tid + 256 * q;
      uint32_t v = 0;
      if (e < 3 * F) {
        const int off = e % F, k = off / CPW, ch = off % CPW;
        const int64_t tok = tb + tj + k;
        const int ic = cg * CPW + ch;
        if (tj + k < t1) {
          if (q < F / 256) v = Raw<T>::dt(a, tok * a.D + ic);
          else if (q < 2 * F / 256) v = Raw<T>::u(a, tok * a.D + ic);
          else v = Raw<T>::z(a, tok * 2 * a.D + a.D + ic);
        }
      } else if (e < ST) {
        const int off = e - 3 * F, k = off / (2 * N), nn = off % (2 * N);
        if (tj + k < t1) v = __float_as_uint(a.bc[(tb + tj + k) * 2 * N + nn]);
      }
      pf[q] = v;
    }
  };
  const float *s_dt = st_s, *s_u = st_s + F, *s_z = st_s + 2 * F, *s_bc = st_s + 3 * F;
  fetch(0);
  for (int jb = 0; jb < nsb; ++jb) {
    // LDS-only barriers: the y stores of the previous sub-block stay in flight
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      st_s[tid + 256 * q] = q < F / 256 ? Raw<T>::dt_f(pf[q])
                            : q < 2 * F / 256 ? Raw<T>::u_f(pf[q])
                            : q < 3 * F / 256 ? Raw<T>::z_f(pf[q]) : __uint_as_float(pf[q]);
    lds_barrier();
    if (jb + 1 < nsb) fetch(jb + 1);
    const int tj = t0 + jb * kGS;
#pragma unroll 4
    for (int k = 0; k < kGS; ++k) {
      if (tj + k < t1) {
        const float dtv = s_dt[k * CPW + c], uv = s_u[k * CPW + c];
        float Bv[S], Cv[S];
        lds_vec<S>(s_bc + k * 2 * N + n0, Bv);
        lds_vec<S>(s_bc + k * 2 * N + N + n0, Cv);
        float yp = 0.f;
#pragma unroll
        for (int q = 0; q < S; ++q) {
          const float av = exp2_hw(dtv * A2[q]);
          const float bb = (ZOH ? expm1_f(dtv * An[q]) * iA[q] : dtv) * Bv[q];
          h[q] = __builtin_fmaf(av, h[q], bb * uv);
          yp = __builtin_fmaf(Cv[q], h[q], yp);
        }
        const float ys = sum_group<G>(yp);
        if (j == 0)
          io<T>::st((T *)a.y + (tb + tj + k) * a.D + i,
                    __builtin_fmaf(Dv, uv, ys) * silu_f(s_z[k * CPW + c]));
      }
    }
  }
}

template <typename T, int N, bool ZOH>
hipError_t launch_n(const ScanArgs &a, hipStream_t s) {
  const int nr = (a.L + kGR - 1) / kGR;
  constexpr int G = N / states_per_lane<N>();
  const unsigned grid = (unsigned)((int64_t)a.B * nr * (a.D / (256 / G)));
  hipLaunchKernelGGL((scanN_transfer_kernel<T, N, ZOH>), dim3(grid), dim3(256), 0, s, a, nr);
  const int64_t nc = (int64_t)a.B * a.D * N;
  hipLaunchKernelGGL((scanN_carry_kernel<N>), dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, a, nr);
  hipLaunchKernelGGL((scanN_replay_kernel<T, N, ZOH>), dim3(grid), dim3(256), 0, s, a, nr);
  return hipGetLastError();
}

template <typename T, bool ZOH>
hipError_t dispatch_n(const ScanArgs &a, hipStream_t s) {
  switch (a.N) {
    case 8: return launch_n<T, 8, ZOH>(a, s);
    case 32: return launch_n<T, 32, ZOH>(a, s);
    case 64: return launch_n<T, 64, ZOH>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool scan_n_supported(int N) { return N == 8 || N == 32 || N == 64; }
int scan_n_ranges(int L) { return (L + kGR - 1) / kGR; }

hipError_t launch_scan_n(mm_dtype dt, const ScanArgs &a, hipStream_t s) {
  if (dt == MM_BF16) return a.zoh ? dispatch_n<bf16_t, true>(a, s) : dispatch_n<bf16_t, false>(a, s);
  return a.zoh ? dispatch_n<float, true>(a, s) : dispatch_n<float, false>(a, s);
}

}  // namespace mm
