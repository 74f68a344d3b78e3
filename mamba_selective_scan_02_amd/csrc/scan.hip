// Selective scan + D feed-through + SiLU(z) gate + final SSM state.
//
// Jamba analysis page, "The Mamba Layer": every channel i runs its own scalar SSM with a
// diagonal A[i, :] over N states ("From scalar SSM to vector processing"); ZOH gives
// Abar = exp(dt A) (ZOH equation); the discrete recurrence h_t = Abar h_{t-1} + Bbar u_t,
// y_t = C_t h_t (recurrence equation); the continuous model's D u feed-through (continuous
// SSM equation). Bbar = dt B by default, or the page's ZOH form expm1(dt A)/A B with
// MM_FLAG_ZOH_B. Gate: y <- y * SiLU(z) (Mamba-1 block).
//
// The SSM input u = SiLU(conv1d(x) + b) is recomputed here in fp32 from x (K taps per token)
// instead of being read back rounded, so the scan sees u at full precision while reading no
// more bytes (x instead of u). dt is read in fp32.
//
// Two kernels, both one pass over the sequence in time order with exactly one exp per
// (token, channel, state), as in the recurrence itself:
//  * scan_seq_kernel: one lane per (sequence, channel), all N = 16 states in VGPRs, B_t / C_t
//    wave-uniform. For many sequences (>= 2048 waves of 64 channels).
//  * scan_lanes_kernel: lanes over (channel, group of states), for few sequences at long L
//    (batch 1 of 8192 channels has only 131072 (channel, state) chains: exactly two per lane
//    of the chip at one wave per SIMD, one per lane at two). See the comment above it.
#include "common.h"
#include "kernels.h"

namespace mm {
namespace {

constexpr int kN = 16;

template <typename T, bool ZOH, int K>
__global__ __launch_bounds__(64) void scan_seq_kernel(ScanArgs a) {
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
  const float *dp = a.delta + (int64_t)b * a.L * a.D + i;
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
    const float dt = dp[(int64_t)t * a.D];
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
// scan_lanes_kernel: one pass in time order, lanes over (channel, state group).
//
// A workgroup owns kLC = 32 channels of one sequence and all N of their states: W waves of 64
// lanes, lane (c = lane % 32, half = lane / 32) of wave w holding the S = N / (2 W) consecutive
// states [S (2 w + half), +S) of channel c in VGPRs (d_state 16: W = 8 waves of one state per
// lane). At batch 1 and d_inner 8192 that is 256 workgroups, one per CU, two waves per SIMD
// (131072 (channel, state) chains: two per lane of the chip), and no time-parallel split: no
// second pass, no carry composition. The sequence is walked in blocks of kLT = 32 tokens, with
// one workgroup barrier per block and three phases in flight:
//   P(j + 1)  prep: thread (channel pair c2, token group g) forms u = SiLU(conv1d(x) + b) in
//             fp32 (the K - 1 rows before the block come from a halo kept in LDS, never
//             re-read), dt, dt*u (u for ZOH), D*u and SiLU(z) once per (token, channel);
//   S(j)      scan: per token each lane reads (dt, dt*u) of its channel and B_t, C_t of its
//             states from LDS (broadcast reads, one token ahead of use), updates its states
//             and forms C . h over them; the two halves of a wave (the same channel, other
//             states) are added by one v_permlane32_swap per token pair, and each wave's
//             partial sum goes to LDS;
//   Y(j - 1)  output: the prep thread adds the W waves' partial sums in a fixed order, applies
//             D u and the gate, and stores two channels (4 bytes) per token.
// x, z and dt rows of block j + 2 and the B|C rows of block j + 1 are loaded by direct-to-LDS
// 16-byte loads while block j is scanned.
//
// Paired decay (S >= 2, d_state 32 / 64): when every lane's states have
// A[i, n0 + k] = A[i, n0] + k delta_i (checked in the kernel; the configs' A = -(n + 1) has
// delta = -1), exp(dt A[i, n0 + k]) is formed as exp(dt A[i, n0]) exp(dt delta_i)^k with
// exp(dt delta_i) computed once per (token, channel) in the prep: one exp per lane and token
// instead of S. ScanArgs::general_a turns the check off (every exp(dt A) evaluated directly);
// ZOH always evaluates them directly.
constexpr int kLC = 32, kLT = 32;

// waves per workgroup: 8 (two per SIMD), or N / 2 below that; fp32 I/O at d_state 64 takes 4
// (its staged fp32 rows would not fit 160 KB of LDS beside 8 waves' partial sums)
template <typename T, int N>
constexpr int lane_waves() {
  return (N == 64 && sizeof(T) == 4) ? 4 : (N / 2 < 8 ? N / 2 : 8);
}

template <typename T, int N>
struct LaneSmem {
  static constexpr int W = lane_waves<T, N>(), S = N / (2 * W);
  T xs[2][kLT][kLC];             // staged x rows (blocks j + 1, j + 2)
  T zs[2][kLT][kLC];             // staged z rows
  float ds[2][kLT][kLC];         // staged dt rows
  float bcs[2][kLT][2 * N];      // staged B | C rows (blocks j, j + 1)
  float halo[2][3][kLC];         // the 3 x rows before a block, as fp32
  float2 pd[2][kLT][kLC];        // (dt, dt*u or u) per (token, channel)
  float pe[S >= 2 ? 2 : 1][kLT][S >= 2 ? kLC : 1];   // exp(dt delta) (paired decay)
  float2 eg[2][kLT][kLC];        // (D*u, SiLU(z))
  float yp[2][W][kLT][kLC];      // each wave's partial C . h
};

template <typename T, bool ZOH, int K, int N, bool PAIRED>
__device__ __forceinline__ void lanes_body(const ScanArgs &a, LaneSmem<T, N> &sm, int b,
                                           int ch0) {
  constexpr int W = LaneSmem<T, N>::W, S = LaneSmem<T, N>::S;
  constexpr int TPT = kLT * 16 / (64 * W);     // tokens per prep / output thread (1 or 2)
  static_assert(!PAIRED || S >= 2, "paired decay needs two states per lane");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // scan roles
  const int c = lane & 31, half = lane >> 5, n0 = (2 * wv + half) * S;
  const int ch = ch0 + c;
  // prep / output roles: channels 2 c2, 2 c2 + 1 at tokens TPT g .. TPT g + TPT - 1
  const int c2 = tid & 15, g = tid >> 4;
  const int nb = (a.L + kLT - 1) / kLT;
  const int Lm1 = a.L - 1;
  const int64_t row = 2LL * a.D;
  const T *xzb = (const T *)a.xz + (int64_t)b * a.L * row;
  const float *db = a.delta + (int64_t)b * a.L * a.D;
  const float *bcb = a.bc + (int64_t)b * a.L * 2 * N;
  T *yb = (T *)a.y + (int64_t)b * a.L * a.D;

  float Av[S], A2[S], iA[S], h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float An = a.A[(int64_t)ch * N + n0 + s];
    Av[s] = An;
    A2[s] = An * kLog2e;
    iA[s] = 1.0f / An;
    h[s] = (a.state_valid && a.state) ? a.state[((int64_t)b * a.D + ch) * N + n0 + s] : 0.f;
  }
  // prep constants of the two channels
  float wc[2][K], cb[2], Dv[2], dl2[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int ce = ch0 + 2 * c2 + e;
#pragma unroll
    for (int k = 0; k < K; ++k) wc[e][k] = io<T>::cvt(((const T *)a.conv_w)[(int64_t)ce * K + k]);
    cb[e] = a.conv_b ? io<T>::cvt(((const T *)a.conv_b)[ce]) : 0.f;
    Dv[e] = a.Dskip[ce];
    dl2[e] = PAIRED ? (a.A[(int64_t)ce * N + 1] - a.A[(int64_t)ce * N]) * kLog2e : 0.f;
  }

  // ---- direct-to-LDS staging (one 16-byte load per lane and wave-round)
  auto stage_xzd = [&](int j) {
    const int T0 = j * kLT;
    const int buf = j & 1;
    if (sizeof(T) == 2) {
      // x, then z: 32 rows of 64 B each = 2 wave-rounds each (4 lanes per row, 16 rows)
#pragma unroll
      for (int q = wv; q < 4; q += W) {
        const int r = (q & 1) * 16 + (lane >> 2);
        const int t = min(T0 + r, Lm1);
        const T *src = xzb + (int64_t)t * row + ch0 + (lane & 3) * 8 + (q >= 2 ? a.D : 0);
        T *dst = q < 2 ? &sm.xs[buf][(q & 1) * 16][0] : &sm.zs[buf][(q & 1) * 16][0];
        dma16_opaque(src, lds_addr(dst));
      }
    } else {
      // fp32: rows of 128 B, 8 lanes per row, 8 rows per wave-round; 4 rounds for x, 4 for z
#pragma unroll
      for (int q = wv; q < 8; q += W) {
        const int r = (q & 3) * 8 + (lane >> 3);
        const int t = min(T0 + r, Lm1);
        const T *src = xzb + (int64_t)t * row + ch0 + (lane & 7) * 4 + (q >= 4 ? a.D : 0);
        T *dst = q < 4 ? &sm.xs[buf][(q & 3) * 8][0] : &sm.zs[buf][(q & 3) * 8][0];
        dma16_opaque(src, lds_addr(dst));
      }
    }
    // dt: rows of 128 B, 8 rows per wave-round, 4 rounds
#pragma unroll
    for (int q = wv; q < 4; q += W) {
      const int r = q * 8 + (lane >> 3);
      const int t = min(T0 + r, Lm1);
      dma16_opaque(db + (int64_t)t * a.D + ch0 + (lane & 7) * 4, lds_addr(&sm.ds[buf][q * 8][0]));
    }
  };
  auto stage_bc = [&](int j) {
    // kLT rows of 2N floats = 256 N bytes = N / 4 wave-rounds of 1 KB
    constexpr int rounds = N / 4;
    constexpr int rowchunks = 2 * N / 4;                 // 16-byte chunks per row
    const int T0 = j * kLT;
    float *dst0 = &sm.bcs[j & 1][0][0];
#pragma unroll
    for (int q = wv; q < rounds; q += W) {
      const int e = q * 64 + lane;                       // chunk index within the block
      const int r = e / rowchunks, cc = e % rowchunks;
      const int t = min(T0 + r, Lm1);
      dma16_opaque(bcb + (int64_t)t * 2 * N + cc * 4, lds_addr(dst0 + q * 256));
    }
  };

  // ---- phases
  auto prep = [&](int j) {
    const int T0 = j * kLT, buf = j & 1;
    constexpr int NR = TPT + 3;
    // x rows TPT g - 3 .. TPT g + TPT - 1 of the block for both channels (negative rows from
    // the halo)
    float xw[2][NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int br = TPT * g - 3 + r;
      if (br >= 0) {
        if (sizeof(T) == 2) {
          const uint32_t v = *(const uint32_t *)&sm.xs[buf][br][2 * c2];
          xw[0][r] = lo_bf(v);
          xw[1][r] = hi_bf(v);
        } else {
          const float2 v = *(const float2 *)&sm.xs[buf][br][2 * c2];
          xw[0][r] = v.x;
          xw[1][r] = v.y;
        }
      } else {
        const float2 v = *(const float2 *)&sm.halo[buf][3 + br][2 * c2];
        xw[0][r] = v.x;
        xw[1][r] = v.y;
      }
    }
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      const int tt = TPT * g + e;
      // the last 3 rows of this block are the next block's halo
      if (tt >= kLT - 3)
        *(float2 *)&sm.halo[buf ^ 1][tt - (kLT - 3)][2 * c2] = make_float2(xw[0][3 + e], xw[1][3 + e]);
      const bool valid = T0 + tt < a.L;
      float zv[2];
      if (sizeof(T) == 2) {
        const uint32_t v = *(const uint32_t *)&sm.zs[buf][tt][2 * c2];
        zv[0] = lo_bf(v);
        zv[1] = hi_bf(v);
      } else {
        const float2 v = *(const float2 *)&sm.zs[buf][tt][2 * c2];
        zv[0] = v.x;
        zv[1] = v.y;
      }
      const float2 dv = *(const float2 *)&sm.ds[buf][tt][2 * c2];
      const float dts[2] = {valid ? dv.x : 0.f, valid ? dv.y : 0.f};
      float4 o, q;
      float pz[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float acc = cb[cc];
#pragma unroll
        for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wc[cc][k], xw[cc][e + 4 - K + k], acc);
        const float u = silu_f(acc);
        // Past the end only dt is zeroed: the step is then the identity (exp(0 A) = 1, no
        // input), and those tokens' outputs are never stored. Staged rows there hold copies of
        // row L - 1, so u and z stay finite.
        const float dt = dts[cc];
        const float2 od = make_float2(dt, ZOH ? u : dt * u);
        const float2 oq = make_float2(Dv[cc] * u, silu_f(zv[cc]));
        if (cc == 0) {
          o.x = od.x; o.y = od.y; q.x = oq.x; q.y = oq.y;
        } else {
          o.z = od.x; o.w = od.y; q.z = oq.x; q.w = oq.y;
        }
        pz[cc] = PAIRED ? exp2_hw(dt * dl2[cc]) : 0.f;
      }
      *(float4 *)&sm.pd[buf][tt][2 * c2] = o;
      *(float4 *)&sm.eg[buf][tt][2 * c2] = q;
      if (PAIRED) *(float2 *)&sm.pe[buf][tt][2 * c2] = make_float2(pz[0], pz[1]);
    }
  };

  auto output = [&](int j) {
    const int T0 = j * kLT, buf = j & 1;
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      const int tt = TPT * g + e;
      float2 s = *(const float2 *)&sm.yp[buf][0][tt][2 * c2];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float2 v = *(const float2 *)&sm.yp[buf][w][tt][2 * c2];
        s.x += v.x;
        s.y += v.y;
      }
      const float4 q = *(const float4 *)&sm.eg[buf][tt][2 * c2];
      const float y0 = (s.x + q.x) * q.y, y1 = (s.y + q.z) * q.w;
      if (T0 + tt < a.L) {
        T *dst = yb + (int64_t)(T0 + tt) * a.D + ch0 + 2 * c2;
        if (sizeof(T) == 2)
          *(uint32_t *)dst = pack_bf2(y0, y1);
        else
          *(float2 *)dst = make_float2(y0, y1);
      }
    }
  };

  // operands of one token for this lane
  struct Tok {
    float2 p;
    float e1;
    float B[S], C[S];
  };
  auto load_tok = [&](int buf, int t, Tok &k) {
    k.p = sm.pd[buf][t][c];
    k.e1 = PAIRED ? sm.pe[buf][t][c] : 0.f;
    const float *Bt = &sm.bcs[buf][t][n0];
    const float *Ct = Bt + N;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      k.B[s] = Bt[s];
      k.C[s] = Ct[s];
    }
  };
  auto step = [&](const Tok &k) -> float {
    float dA = 0.f, yy = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (ZOH) {
        const float em1 = expm1_f(k.p.x * Av[s]);
        h[s] = __builtin_fmaf(em1 + 1.0f, h[s], em1 * iA[s] * k.B[s] * k.p.y);
      } else {
        dA = (PAIRED && s > 0) ? dA * k.e1 : exp2_hw(k.p.x * A2[s]);
        h[s] = __builtin_fmaf(dA, h[s], k.p.y * k.B[s]);
      }
      yy = s == 0 ? k.C[0] * h[0] : __builtin_fmaf(k.C[s], h[s], yy);
    }
    return yy;
  };
  auto scan = [&](int j) {
    const int buf = j & 1;
    Tok cur[2], nxt[2];
    load_tok(buf, 0, cur[0]);
    load_tok(buf, 1, cur[1]);
#pragma unroll
    for (int t = 0; t < kLT; t += 2) {
      if (t + 2 < kLT) {   // next pair's operands in flight while this pair is computed
        load_tok(buf, t + 2, nxt[0]);
        load_tok(buf, t + 3, nxt[1]);
      }
      const float q0 = step(cur[0]);
      const float q1 = step(cur[1]);
      // lanes c (half 0) and c + 32 (half 1) hold the same channel's other states: after the
      // swap, half 0 has both halves' terms of token t, half 1 both of token t + 1
      const auto w2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(q0), __float_as_uint(q1),
                                                       false, false);
      sm.yp[buf][wv][t + half][c] = __uint_as_float(w2[0]) + __uint_as_float(w2[1]);
      if (t + 2 < kLT) {
        cur[0] = nxt[0];
        cur[1] = nxt[1];
      }
    }
  };

  // ---- prologue: stage blocks 0 (B|C), 0 and 1 (x, z, dt); halo of block 0 = the carried
  // conv state (oldest first) or zeros; prep of block 0
  stage_bc(0);
  stage_xzd(0);
  if (nb > 1) stage_xzd(1);
  if (tid < 3 * kLC) {
    const int r = tid / kLC, cc = tid % kLC;   // halo row r <-> token r - 3
    const int si = r - (3 - (K - 1));          // index into the K - 1 state entries
    float v = 0.f;
    if (si >= 0 && a.conv_valid && a.conv_state)
      v = io<T>::cvt(((const T *)a.conv_state)[((int64_t)b * a.D + ch0 + cc) * (K - 1) + si]);
    sm.halo[0][r][cc] = v;
  }
  wait_vmem_all();
  lds_barrier();
  prep(0);
  for (int j = 0; j < nb; ++j) {
    wait_vmem_all();   // this wave's staged rows of blocks j + 1 (x, z, dt) and j (B|C)
    lds_barrier();     // ... everyone's; P(j), S(j - 1) are complete
    if (j + 2 < nb) stage_xzd(j + 2);
    if (j + 1 < nb) stage_bc(j + 1);
    if (j > 0) output(j - 1);
    if (j + 1 < nb) prep(j + 1);
    scan(j);
  }
  wait_vmem_all();
  lds_barrier();
  output(nb - 1);
  if (a.state) {
#pragma unroll
    for (int s = 0; s < S; ++s) a.state[((int64_t)b * a.D + ch) * N + n0 + s] = h[s];
  }
}

template <typename T, bool ZOH, int K, int N>
__global__ __launch_bounds__((64 * lane_waves<T, N>())) void scan_lanes_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) LaneSmem<T, N> sm;
  constexpr int S = LaneSmem<T, N>::S;
  const int groups = a.D / kLC;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = gid / groups, ch0 = (gid % groups) * kLC;
  if constexpr (ZOH || S < 2) {
    lanes_body<T, ZOH, K, N, false>(a, sm, b, ch0);
  } else {
    // paired decay: every lane's S states in arithmetic progression with the channel's step
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ch = ch0 + (lane & 31), n0 = (2 * wv + (lane >> 5)) * S;
    const float *Ar = a.A + (int64_t)ch * N;
    const float dl = Ar[1] - Ar[0];
    int ok = !a.general_a;
#pragma unroll
    for (int s = 1; s < S; ++s) ok &= (Ar[n0 + s] - Ar[n0] == (float)s * dl);
    if (__syncthreads_and(ok))
      lanes_body<T, ZOH, K, N, true>(a, sm, b, ch0);
    else
      lanes_body<T, ZOH, K, N, false>(a, sm, b, ch0);
  }
}

template <typename T, int K>
hipError_t dispatch_lanes_k(const ScanArgs &a, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)a.B * (a.D / kLC));
#define MM_LANES(NN)                                                                         \
  if (a.N == NN) {                                                                           \
    constexpr int thr = 64 * lane_waves<T, NN>();                                            \
    if (a.zoh)                                                                               \
      hipLaunchKernelGGL((scan_lanes_kernel<T, true, K, NN>), dim3(blocks), dim3(thr), 0, s, a); \
    else                                                                                     \
      hipLaunchKernelGGL((scan_lanes_kernel<T, false, K, NN>), dim3(blocks), dim3(thr), 0, s, a); \
    return hipGetLastError();                                                                \
  }
  MM_LANES(8)
  MM_LANES(16)
  MM_LANES(32)
  MM_LANES(64)
#undef MM_LANES
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------
// scan_twopass_kernel: time-parallel scan for d_state 16 at few sequences (the 128K prefill).
//
// A workgroup owns kCh = 32 channels of one sequence and walks the sequence in blocks of
// kW * kS = 96 tokens; wave w owns the kS-token segment w of every block. 12 waves of 8
// tokens give three waves per SIMD at batch 1 (256 workgroups): the VALU and v_exp_f32 issue
// rates are lower at two, and at four the 128 VGPRs a wave may then hold do not keep the
// segment's exp(dt A) without spilling. Lane l works on channel l / 2 and the 8 states
// 8 (l % 2) .. +7 (B_t / C_t reads from LDS serve 8 updates):
//  0. The segment's B|C rows, its x rows (with the 3 conv-window rows before it), z and dt
//     rows were loaded into the wave's LDS rows with direct-to-LDS 16-byte loads while the
//     previous block was computed (blocks inside the sequence take each lane's byte offsets
//     from a table formed once; edge blocks clamp rows into the sequence).
//  1. Prep: lane l takes channel l / 2 and the segment's tokens kS/2 (l % 2) .. +kS/2-1:
//     u = SiLU(conv1d(x) + b), dt and dt*u go to the wave's LDS rows; D*u and SiLU(z) of
//     those tokens stay in the lane's registers for step 4 (the wave waits on its own loads
//     only; no workgroup barrier).
//  2. Local pass: the segment is scanned from h = 0, keeping exp(dt A) of every (token, state)
//     in VGPRs (one exp per element, as in the sequential recurrence).
//  3. Compose: the segment's transfer h -> P h + S (local end state S, decay
//     P = exp(A sum dt)) goes to LDS as S and the segment's sum dt per channel (barrier).
//     Thread i then owns one (channel, state) chain: it forms each segment's P from its sum dt
//     and applies the segments' transfers in order to
//     the block's carry-in with the page's associative operator ("Parallel training via the
//     parallel scan": (a, b) then (c, d) gives (ac, ad + b) for h -> a h + b), writing each
//     segment's h_in over its S (barrier), and keeps the result as the next block's carry-in.
//  4. Replay from the true h_in with the stored exp(dt A); y_t = C_t . h_t as two half-sums
//     per channel, one per lane; the halves meet by a DPP lane swap, each lane keeping the
//     tokens of its prep, and y = (y_ssm + D u) SiLU(z) goes out.
// First-order Bbar only (the ZOH form would need expm1(dt A) and 1 / A in VGPRs besides).
// Paired decay (as in the lane kernel; off with ScanArgs::general_a): when
// A[i, 8 p + k] = A[i, 8 p] + k delta_i for every lane, the local pass forms a lane's 8
// decays as exp(dt A[i, 8 p]) times powers of exp(dt delta_i): 2 exps per lane and token
// instead of 8.
// Fused dt_proj (ScanArgs::dtlow set): instead of staging dt rows, the workgroup forms the
// next block's dt after each replay from the normalised dt_low with split-precision MFMAs
// (dt_phase below) and a third barrier hands it to the prep.
constexpr int kCh = 32, kW = 12, kS = 8, kG = 8, kBlk = kW * kS;
constexpr int kHalf = kS / 2;             // tokens per lane in the prep and the output
constexpr int kHalo = 3;                  // x rows before the segment (conv window, K - 1 <= 3)
constexpr int kXSeg = kS + kHalo;         // x rows a segment needs: halo + segment
constexpr int kXZR = 16;                  // staged x / z rows per wave: one 16-byte slot per lane
static_assert(kXSeg <= kXZR && kS <= kXZR, "a wave's x and z rows fit one wave-load");
// The two lanes of a channel read staged rows kHalf = 4 apart in the same instruction; the rows
// are placed so that the two lane halves hit different LDS banks:
//  * x (64-byte rows k <-> token T0w - 3 + k): lane half p reads rows 4 p .. 4 p + 6, kept at
//    slots 9 p + (k - 4 p) (rows 0..6 at slots 0..6, rows 4..10 again at slots 9..15);
//  * z (64-byte rows k <-> token T0w + k): row k at slot k + (k >= 4), i.e. row 4 p + e at
//    slot 5 p + e;
//  * dt (128-byte rows): row k at slot k ^ ((k >> 2) & 1), so rows e and 4 + e differ in parity.
static_assert(kS == 8 && kHalf == 4 && kHalo == 3, "the staged-row placement assumes these");
__device__ __forceinline__ int x_slot_row(int s) { return s < 7 ? s : (s < 9 ? 6 : s - 5); }
__device__ __forceinline__ int z_slot_row(int s) { return s < 4 ? s : min(s - 1, 7); }
__device__ __forceinline__ int d_slot_row(int s) { return s ^ ((s >> 2) & 1); }
constexpr int kChains = kCh * kN;         // (channel, state) chains of a workgroup
static_assert(kChains == 512 && kW * 64 >= kChains, "chain threads map onto 512 agg floats");
static_assert(kW * kS * 64 <= 65536 && kW * 2 * 64 * 16 <= 65536, "LDS offsets fit 16 bits");

constexpr int kFR = 256;                  // dt_rank of the fused dt_proj
constexpr int kFK = kFR / 32;             // its k-steps (16x16x32 MFMAs per plane)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename T, bool FDT>
struct TwoPassSmem {
  // bf16 I/O stages x, z and dt through LDS; fp32 I/O (small problems) reads them from
  // global memory in the prep, which keeps its LDS within 160 KB
  static constexpr bool kStage = sizeof(T) == 2;
  static constexpr int kXR = kStage ? kXZR : 1, kZR = kStage ? kS : 1;
  // per-wave staging (written by async loads); B|C double-buffered. Every lane of a wave
  // issues each load (no divergent branch around them): the x and z loads fill 16 rows, the
  // rows past those the segment needs repeating its last row
  float bc[2][kW][kS][2 * kN];
  T x[kW][kXR][kCh];
  T z[kW][kXR][kCh];
  float d[kW][kZR][kCh];      // staged dt rows, or dt formed in the workgroup (fused dt_proj)
  // prep output: (dt, dt*u) per (token, channel) of each wave's segment; rows padded by one
  // element so that the rows of the two lanes of a channel fall in different LDS banks
  float2 pd[kW][kS][kCh + 1];
  // per segment and lane, 16-byte slots [wave][S0..3, S4..7][lane]: the local end states S
  // (overwritten by the segments' true start states); and per segment and channel, the sum
  // of dt over the segment, from which the chain threads form the decays P = exp(A sum dt)
  float4 agg[kW][2][64];
  float sdt[kW][kCh];
  // per channel: conv taps (K) | conv bias, D, -, -; and A log2(e) as [half][lane] 16-byte
  // slots (lane 2 c + p holds states 8 p + 4 half .. +3 of channel c): the per-block reads are
  // lane-contiguous
  float4 cst[2][kCh];
  float4 a2[2][2 * kCh];
  // fused dt_proj: the workgroup's W_dt rows (16-byte slot c of row r at slot c ^ (r % 16), so
  // that a fragment read of 16 rows is bank-conflict free), their biases, and the sink of the
  // dt_low prefetch (written, never read)
  bf16_t wdt[FDT ? kCh : 1][FDT ? kFR : 8];
  float dtb[FDT ? kCh : 4];
  float pf[FDT ? kW : 1][64];
  // bf16, unfused: each lane's byte offsets of its B|C, x, z and dt staging loads for blocks
  // whose rows all lie inside the sequence (formed once; the edge blocks clamp rows instead)
  static constexpr bool kOffTab = kStage && !FDT;
  uint4 doff[kOffTab ? kW : 1][64];
};

template <typename T, int K, bool PAIRED, bool FDT>
__device__ __forceinline__ void twopass_body(const ScanArgs &a, TwoPassSmem<T, FDT> &sm, int b,
                                             int ch0) {
  constexpr bool kStage = TwoPassSmem<T, FDT>::kStage;
  static_assert(!FDT || kStage, "the fused dt_proj is built for bf16 I/O");
  constexpr int xrow_chunks = kCh * sizeof(T) / 16;    // 16-byte chunks per staged x/z row
  constexpr uint32_t kPdRow = (kCh + 1) * sizeof(float2), kBcRow = 2 * kN * sizeof(float);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  // chain thread tid (waves 0-7) <-> publishing lane ql = (tid >> 2) & 63 (channel ql / 2,
  // state half ql & 1), state j = 4 (tid >> 8) + (tid & 3) of that half: its S of segment w
  // is float w * 512 + tid of agg (conflict-free)
  const bool chain = wv < kChains / 64;
  float carry = 0.f;
  if (chain && a.state_valid && a.state) {
    const int tid = threadIdx.x, ql = (tid >> 2) & 63, qj = 4 * ((tid >> 8) & 1) + (tid & 3);
    carry = a.state[((int64_t)b * a.D + ch0 + (ql >> 1)) * kN + kG * (ql & 1) + qj];
  }
  const float dl2 = PAIRED ? (a.A[(ch0 + (threadIdx.x & 63) / 2) * kN + kG * (threadIdx.x & 1) + 1] -
                              a.A[(ch0 + (threadIdx.x & 63) / 2) * kN + kG * (threadIdx.x & 1)]) * kLog2e
                           : 0.f;

  const int64_t row = 2LL * a.D;
  const T *xzb = (const T *)a.xz + (int64_t)b * a.L * row;
  const float *db = a.delta + (int64_t)b * a.L * a.D;
  const float *bcb = a.bc + (int64_t)b * a.L * 2 * kN;
  T *yb = (T *)a.y + (int64_t)b * a.L * a.D;
  const int nblocks = (a.L + kBlk - 1) / kBlk;
  const int Lm1 = a.L - 1;

  // Issue the direct-to-LDS loads of this wave's segment of block `blk` (lane = this lane).
  // Rows outside [0, L) read the nearest valid row (every address is valid; prep and the scan
  // ignore those rows).
  constexpr bool kOffTab = TwoPassSmem<T, FDT>::kOffTab;
  // this lane's staging offsets for a block inside the sequence: B|C row lane / 8 (16 bytes at
  // 16 (lane % 8)), x row x_slot_row(sl) from the third row before the segment, z row
  // z_slot_row(sl), dt row d_slot_row(lane / 8) (sl = lane / xrow_chunks)
  auto interior_offsets = [&](int lane) -> uint4 {
    const int sl = lane / xrow_chunks;
    const uint32_t rowb = (uint32_t)row * (uint32_t)sizeof(T);
    const uint32_t cb16 = (uint32_t)((lane % xrow_chunks) * 16);
    return make_uint4((uint32_t)((lane >> 3) * 2 * kN + 4 * (lane & 7)) * 4u,
                      (uint32_t)x_slot_row(sl) * rowb + cb16, (uint32_t)z_slot_row(sl) * rowb + cb16,
                      (uint32_t)d_slot_row(lane >> 3) * (uint32_t)a.D * 4u + (uint32_t)((lane & 7) * 16));
  };
  auto stage = [&](int blk, float (*bcdst)[2 * kN], int lane, uint4 off) {
    // wave-uniform bases (SGPRs) and 32-bit lane offsets, so that no 64-bit address lives in
    // VGPRs across the block; rows outside [0, L) are clamped into it
    const int T0w = blk * kBlk + wv * kS;
    if (kOffTab && T0w >= kHalo && T0w + kS - 1 <= Lm1) {   // wave-uniform: no row is clamped
      dma16_opaque_so(bcb + (int64_t)T0w * 2 * kN, off.x, lds_addr(&bcdst[0][0]));
      dma16_opaque_so(xzb + (int64_t)(T0w - kHalo) * row + ch0, off.y, lds_addr(&sm.x[wv][0][0]));
      dma16_opaque_so(xzb + (int64_t)T0w * row + a.D + ch0, off.z, lds_addr(&sm.z[wv][0][0]));
      dma16_opaque_so(db + (int64_t)T0w * a.D + ch0, off.w, lds_addr(&sm.d[wv][0][0]));
      return;
    }
    const int tb = min(T0w, Lm1);                 // first staged row of B|C, z, dt
    // B|C: kS rows x 128 B = kS / 8 wave-loads, 8 lanes per row; slots 0-3 B, 4-7 C
#pragma unroll
    for (int i = 0; i < kS / 8; ++i) {
      const int r = min(T0w + i * 8 + (lane >> 3), Lm1) - tb;
      dma16_opaque_so(bcb + (int64_t)tb * 2 * kN, (uint32_t)(r * 2 * kN + 4 * (lane & 7)) * 4u,
                      lds_addr(&bcdst[i * 8][0]));
    }
    if (!kStage) return;
    // x: slot s holds row x_slot_row(s) <-> token T0w - 3 + row; z: slot s holds row
    // z_slot_row(s) <-> token T0w + row; dt: slot s holds row d_slot_row(s)
    static_assert(!kStage || 64 / xrow_chunks == kXZR, "one wave-load covers kXZR rows");
    const int sl = lane / xrow_chunks;
    const uint32_t rowb = (uint32_t)row * (uint32_t)sizeof(T);
    const uint32_t cb16 = (uint32_t)((lane % xrow_chunks) * 16);
    const int xb = min(max(T0w - kHalo, 0), Lm1);
    const int rx = min(max(T0w - kHalo + x_slot_row(sl), 0), Lm1) - xb;
    dma16_opaque_so(xzb + (int64_t)xb * row + ch0, (uint32_t)rx * rowb + cb16,
                    lds_addr(&sm.x[wv][0][0]));
    const int rz = min(T0w + z_slot_row(sl), Lm1) - tb;
    dma16_opaque_so(xzb + (int64_t)tb * row + a.D + ch0, (uint32_t)rz * rowb + cb16,
                    lds_addr(&sm.z[wv][0][0]));
    if (!FDT) {
      // dt (fp32): kS = 8 rows x 128 B = one wave-load, 8 lanes per row
      const int rd = min(T0w + d_slot_row(lane >> 3), Lm1) - tb;
      dma16_opaque_so(db + (int64_t)tb * a.D + ch0, (uint32_t)rd * (uint32_t)a.D * 4u + (uint32_t)((lane & 7) * 16),
                      lds_addr(&sm.d[wv][0][0]));
    } else {
      // fused dt_proj: touch this segment's dt_low rows (both planes, 512 B per row each) so
      // that the dt phase at the end of the block finds them in L2; lane l reads 4 bytes at
      // row l / 8, byte 64 (l % 8) into the wave's sink
      const uint32_t po = (uint32_t)(min(T0w + (lane >> 3), Lm1) - tb) * (kFR * 2u) + 64u * (lane & 7);
      const int64_t pr = ((int64_t)b * a.L + tb) * kFR;
      dma4_opaque_so(a.dtlow + pr, po, lds_addr(&sm.pf[wv][0]));
      dma4_opaque_so(a.dtlow_lo + pr, po, lds_addr(&sm.pf[wv][0]));
    }
  };

  // Fused dt_proj: dt of block blk into sm.d, in the staged rows' slots, for the prep after the
  // next barrier. Waves 0-5 each form 16 tokens of the block (wave w: tokens 16 w .. +15) for
  // all 32 channels, as two 16 x 16 tiles (lane (tl, g) = (lane % 16, lane / 16) holding token
  // tl and channels 16 nb + 4 g .. +3) that share the dt_low fragments, so that every dt_low
  // row crosses from L2 once per workgroup. The MFMA sequence is dtproj_kernel's (per k-step
  // the low plane, then the high plane, into one fp32 accumulator per tile), which makes dt the
  // same bit for bit.
  auto dt_phase = [&](int blk) {
    constexpr int kTiles = kBlk / 16;              // 16-token tiles per block: waves 0 .. 5
    if (wv >= kTiles) return;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, tl = lane & 15, g = lane >> 4;
    const int t0 = blk * kBlk + 16 * wv;           // wave-uniform
    const int tb = min(t0, Lm1);
    const uint32_t off = (uint32_t)(min(t0 + tl, Lm1) - tb) * (kFR * 2u) + 16u * g;
    const char *hb = (const char *)(a.dtlow + ((int64_t)b * a.L + tb) * kFR);
    const char *lb = (const char *)(a.dtlow_lo + ((int64_t)b * a.L + tb) * kFR);
    uint4 fh[kFK], fl[kFK];
#pragma unroll
    for (int ks = 0; ks < kFK; ++ks) {
      fh[ks] = *(const uint4 *)(hb + (off + 64u * ks));
      fl[ks] = *(const uint4 *)(lb + (off + 64u * ks));
    }
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kFK; ++ks) {
      // both fragments read first, then the low-plane MFMAs, then the high-plane ones
      bf16x8 fw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        fw[nb] = __builtin_bit_cast(bf16x8, *lds_ptr<const uint4>(lds_addr(&sm.wdt[16 * nb + tl][0]) +
                                                                 16u * ((4 * ks + g) ^ tl)));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], __builtin_bit_cast(bf16x8, fl[ks]), acc[nb], 0, 0, 0);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[nb], __builtin_bit_cast(bf16x8, fh[ks]), acc[nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float4 bv = *lds_ptr<const float4>(lds_addr(&sm.dtb[16 * nb + 4 * g]));
      const float4 v = make_float4(softplus_sel(acc[nb][0] + bv.x), softplus_sel(acc[nb][1] + bv.y),
                                   softplus_sel(acc[nb][2] + bv.z), softplus_sel(acc[nb][3] + bv.w));
      *lds_ptr<float4>(lds_addr(&sm.d[2 * wv + (tl >> 3)][d_slot_row(tl & 7)][16 * nb + 4 * g])) = v;
    }
  };

  // y of block b is stored at the start of block b+1, after that block's wait, so the wait
  // for the staged tiles never has to cover freshly issued stores. Lane (c, p) owns tokens
  // kHalf p .. kHalf p + kHalf - 1 of its wave's segment.
  float ypend[kHalf];
  int ypend_t0 = -1;
  auto flush = [&](int c, int p) {
    if (ypend_t0 < 0) return;
    // wave-uniform base and unsigned 32-bit byte offsets (an SGPR base + VGPR offset store)
    char *ybase = (char *)(yb + (int64_t)(ypend_t0 + wv * kS) * a.D);
    const uint32_t off = (uint32_t)(p * kHalf * a.D + ch0 + c) * (uint32_t)sizeof(T);
    const uint32_t step = (uint32_t)a.D * (uint32_t)sizeof(T);
    if (ypend_t0 + kBlk <= a.L) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) io<T>::st((T *)(ybase + (off + i * step)), ypend[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kHalf; ++i)
        if (ypend_t0 + wv * kS + kHalf * p + i < a.L)
          io<T>::st((T *)(ybase + (off + i * step)), ypend[i]);
    }
  };
  auto block = [&](int blk, float (*bc_cur)[kS][2 * kN], float (*bc_nxt)[kS][2 * kN]) {
    const int T0 = blk * kBlk;
    const int T0w = T0 + wv * kS;
    // Lane-dependent values are re-formed per block from an opaque copy of the thread id:
    // held across the block loop (the compiler's choice for loop-invariant values) they
    // would take VGPRs the scan needs.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, c = lane >> 1, p = lane & 1, ch = ch0 + c;
    wait_vmem_all();   // this wave's staged rows (and its older stores) have landed
    flush(c, p);
    uint4 doffs = make_uint4(0u, 0u, 0u, 0u);
    if (kOffTab) doffs = sm.doff[wv][lane];
    // this lane's LDS rows: (dt, dt*u) column, B|C slot
    const uint32_t pdl = lds_addr(&sm.pd[wv][0][c]);
    const uint32_t bcl = lds_addr(&bc_cur[wv][0][kG * p]);
    auto pd_at = [&](int t) -> float2 { return *lds_ptr<const float2>(pdl + t * kPdRow); };
    auto du_at = [&](int t) -> float { return *lds_ptr<const float>(pdl + t * kPdRow + 4); };
    auto b4_at = [&](int t, int q) -> float4 {   // q = 0, 1: B; 2, 3: C
      return *lds_ptr<const float4>(bcl + t * kBcRow + (q & 1) * 16 + (q >> 1) * kN * 4);
    };

    // ---- 1. prep: conv + SiLU, dt, dt*u into LDS; D*u, SiLU(z) kept for the output
    float eDu[kHalf], eg[kHalf];
    {
      // per-channel constants from the workgroup's LDS table
      const float4 c0 = sm.cst[0][c], c1 = sm.cst[1][c];
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      float wc[K];
#pragma unroll
      for (int k = 0; k < K; ++k) wc[k] = cv[k];
      const float cb = cv[4], Dp = cv[5];
      // m: this lane's x row relative to its first window row (token T0w + ts0 + m - 3); e:
      // its e-th token (T0w + ts0 + e); staged slots as placed above
      const int ts0 = kHalf * p;
      constexpr uint32_t kXRow = kCh * sizeof(T);
      const uint32_t xl = lds_addr(&sm.x[wv][0][c]) + 9u * kXRow * p;
      const uint32_t zl = lds_addr(&sm.z[wv][0][c]) + 5u * kXRow * p;
      const uint32_t dle = lds_addr(&sm.d[wv][0][c]) + 5u * kCh * 4 * p;   // even e
      const uint32_t dlo = lds_addr(&sm.d[wv][0][c]) + 3u * kCh * 4 * p;   // odd e
      auto getx = [&](int m) -> float {
        if (kStage) return io<T>::cvt(*lds_ptr<const T>(xl + m * kXRow));
        return io<T>::cvt(xzb[(int64_t)min(T0w + ts0 + m - kHalo, Lm1) * row + ch]);
      };
      auto getz = [&](int e) -> float {
        if (kStage) return io<T>::cvt(*lds_ptr<const T>(zl + e * kXRow));
        return io<T>::cvt(xzb[(int64_t)min(T0w + ts0 + e, Lm1) * row + a.D + ch]);
      };
      auto getd = [&](int e) -> float {
        if (kStage) return *lds_ptr<const float>(((e & 1) ? dlo : dle) + e * kCh * 4);
        return db[(int64_t)min(T0w + ts0 + e, Lm1) * a.D + ch];
      };
      float win[K - 1];
      if (T0w >= kHalo) {   // wave-uniform: every window row is a row of this sequence
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j] = getx(kHalo - (K - 1) + j);
      } else {              // the first segment: rows before token 0 come from the conv state
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
          const int ts = ts0 - (K - 1) + j;       // segment-relative token of this window row
          const int t = T0w + ts;
          float v = 0.f;
          if (t >= 0) {
            v = getx(kHalo - (K - 1) + j);
          } else if (a.conv_valid && a.conv_state) {
            v = io<T>::cvt(((const T *)a.conv_state)[((int64_t)b * a.D + ch) * (K - 1) + (K - 1) + t]);
          }
          win[j] = v;
        }
      }
#pragma unroll
      for (int e = 0; e < kHalf; ++e) {
        const int ts = ts0 + e;
        const bool valid = T0w + ts < a.L;
        const float x = getx(kHalo + e);
        float acc = cb;
#pragma unroll
        for (int j = 0; j < K - 1; ++j) acc = __builtin_fmaf(wc[j], win[j], acc);
        acc = __builtin_fmaf(wc[K - 1], x, acc);
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
        win[K - 2] = x;
        const float u = silu_f(acc);
        // Past the end only dt is zeroed: the step is then the identity (exp(0 A) = 1, no
        // input), and those tokens' outputs are never stored. Staged rows there hold copies of
        // row L-1, so u and z stay finite.
        const float dt = valid ? getd(e) : 0.f;
        *lds_ptr<float2>(pdl + ts * kPdRow) = make_float2(dt, dt * u);
        eDu[e] = Dp * u;
        eg[e] = silu_f(getz(e));
      }
    }
    // the staged x, z, dt rows are consumed once this wave's LDS reads have returned; then the
    // next block's rows may land (B|C is double-buffered)
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0), vmcnt / expcnt unconstrained
    if (blk + 1 < nblocks) stage(blk + 1, bc_nxt[wv], lane, doffs);

    // ---- 2. local pass over this wave's segment
    float A2[kG];
    {
      const float4 q0 = sm.a2[0][lane], q1 = sm.a2[1][lane];
      A2[0] = q0.x; A2[1] = q0.y; A2[2] = q0.z; A2[3] = q0.w;
      A2[4] = q1.x; A2[5] = q1.y; A2[6] = q1.z; A2[7] = q1.w;
    }
    float dA[kS][kG];
    float hl[kG];
    float sumdt = 0.f;
#pragma unroll
    for (int t = 0; t < kS; ++t) {
      const float2 pd = pd_at(t);
      const float dt = pd.x, du = pd.y;
      sumdt += dt;
      const float4 B0 = b4_at(t, 0), B1 = b4_at(t, 1);
      const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
      float e1 = 0.f;
      if (PAIRED) e1 = exp2_hw(dt * dl2);
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        dA[t][j] = (PAIRED && j > 0) ? dA[t][j - 1] * e1 : exp2_hw(dt * A2[j]);
        // the segment starts from h = 0
        hl[j] = t == 0 ? du * Bv[j] : __builtin_fmaf(dA[t][j], hl[j], du * Bv[j]);
      }
    }
    // ---- 3. publish this segment's transfer h -> P h + S, then compose
    sm.agg[wv][0][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
    sm.agg[wv][1][lane] = make_float4(hl[4], hl[5], hl[6], hl[7]);
    if (p == 0) sm.sdt[wv][c] = sumdt;   // the channel's two lanes hold the same sum
    lds_barrier();
    // chain pass: each segment's S becomes its h_in (all reads in flight together, the decays
    // formed from them, then the dependent fmas); the decay exp(A sum dt) is the one the
    // segment's lanes would form (A log2(e) from the same table, the same sum)
    if (chain) {
      const uint32_t al = lds_addr(&sm.agg[0][0][0].x) + 4u * tid;
      constexpr uint32_t kSeg = 2 * 64 * 16;      // bytes per segment in agg
      const int ql = (tid >> 2) & 63;
      const float a2v = (&sm.a2[(tid >> 8) & 1][ql].x)[tid & 3];
      const uint32_t sl = lds_addr(&sm.sdt[0][ql >> 1]);
      float Sw[kW], Pw[kW];
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) {
        Sw[w2] = *lds_ptr<const float>(al + w2 * kSeg);
        Pw[w2] = *lds_ptr<const float>(sl + w2 * kCh * 4);
      }
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) Pw[w2] = exp2_hw(a2v * Pw[w2]);
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) {
        *lds_ptr<float>(al + w2 * kSeg) = carry;
        carry = __builtin_fmaf(Pw[w2], carry, Sw[w2]);
      }
    }
    lds_barrier();
    float h[kG];
    {
      const float4 H0 = sm.agg[wv][0][lane], H1 = sm.agg[wv][1][lane];
      h[0] = H0.x; h[1] = H0.y; h[2] = H0.z; h[3] = H0.w;
      h[4] = H1.x; h[5] = H1.y; h[6] = H1.z; h[7] = H1.w;
    }
    // ---- 4. replay from the true h_in; y from the two half-sums of the channel
    float ys[kHalf];
#pragma unroll
    for (int t = 0; t < kS; ++t) {
      const float4 B0 = b4_at(t, 0), B1 = b4_at(t, 1), C0 = b4_at(t, 2), C1 = b4_at(t, 3);
      const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
      const float Cv[kG] = {C0.x, C0.y, C0.z, C0.w, C1.x, C1.y, C1.z, C1.w};
      const float du = du_at(t);
      float yy = 0.f;
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        h[j] = __builtin_fmaf(dA[t][j], h[j], du * Bv[j]);
        yy = __builtin_fmaf(Cv[j], h[j], yy);
      }
      if (t < kHalf) {
        ys[t] = yy;
      } else {
        // lane p keeps token kHalf p + e: its own half-sum plus the partner lane's half-sum
        const int e = t - kHalf;
        const float keep = p ? yy : ys[e];
        const float send = p ? ys[e] : yy;
        const float other = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
        ypend[e] = (keep + other + eDu[e]) * eg[e];
      }
    }
    ypend_t0 = T0;
    if (FDT && blk + 1 < nblocks) {
      // every wave's prep of this block has read sm.d (first barrier above)
      dt_phase(blk + 1);
      lds_barrier();
    }
  };

  {
    const int tid = threadIdx.x;
    if (tid < kCh) {   // the per-channel constants table (read after the first barrier)
      const int cc = ch0 + tid;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < K; ++k) v[k] = io<T>::cvt(((const T *)a.conv_w)[(int64_t)cc * K + k]);
      v[4] = a.conv_b ? io<T>::cvt(((const T *)a.conv_b)[cc]) : 0.0f;
      v[5] = a.Dskip[cc];
      sm.cst[0][tid] = make_float4(v[0], v[1], v[2], v[3]);
      sm.cst[1][tid] = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (tid < kCh * kN) {   // state n of channel cc: lane 2 cc + n / 8, half (n / 4) % 2
      const int cc = tid / kN, n = tid % kN;
      (&sm.a2[(n >> 2) & 1][2 * cc + (n >> 3)].x)[n & 3] = a.A[(int64_t)ch0 * kN + tid] * kLog2e;
    }
    if (FDT) {
      // W_dt rows of the workgroup's channels (swizzled as above) and their biases
      for (int e = tid; e < kCh * (kFR / 8); e += kW * 64) {
        const int r = e / (kFR / 8), c = e % (kFR / 8);
        *(uint4 *)&sm.wdt[r][8 * (c ^ (r & 15))] = *(const uint4 *)(a.dt_w + (int64_t)(ch0 + r) * kFR + 8 * c);
      }
      if (tid < kCh) sm.dtb[tid] = a.dt_b[ch0 + tid];
    }
    if (kOffTab) sm.doff[wv][tid & 63] = interior_offsets(tid & 63);
    __syncthreads();
    stage(0, sm.bc[0][wv], tid & 63, kOffTab ? sm.doff[wv][tid & 63] : make_uint4(0u, 0u, 0u, 0u));
    if (FDT) {
      dt_phase(0);
      lds_barrier();
    }
  }
  for (int blk = 0; blk < nblocks; ++blk) {
    const bool odd = blk & 1;
    block(blk, odd ? sm.bc[1] : sm.bc[0], odd ? sm.bc[0] : sm.bc[1]);
  }
  {
    const int tid = threadIdx.x;
    flush((tid & 63) >> 1, tid & 1);
    if (chain && a.state) {
      const int ql = (tid >> 2) & 63, qj = 4 * ((tid >> 8) & 1) + (tid & 3);
      a.state[((int64_t)b * a.D + ch0 + (ql >> 1)) * kN + kG * (ql & 1) + qj] = carry;
    }
  }
}

// MODE 0: every workgroup takes the general path (the caller declares A general). Otherwise
// each workgroup checks its channels for paired decay (A given as -(n + 1) per state, or any
// equal step per lane): MODE 1 runs the workgroups that have it (paired path) and MODE 2 those
// that do not (general path), each kernel exiting on the others, so that no kernel holds both
// paths (their registers would add up and spill).
__device__ __forceinline__ bool twopass_paired(const ScanArgs &a, int ch0) {
  // every lane's 8 states in arithmetic progression with the channel's step
  const int lane = threadIdx.x & 63;
  const int ch = ch0 + (lane >> 1), n0 = kG * (lane & 1);
  const float *Ar = a.A + (int64_t)ch * kN;
  const float dl = Ar[1] - Ar[0];
  int ok = 1;
#pragma unroll
  for (int s = 1; s < kG; ++s) ok &= (Ar[n0 + s] - Ar[n0] == (float)s * dl);
  return __syncthreads_and(ok) != 0;
}

template <typename T, int K, int MODE, bool FDT>
__global__ __launch_bounds__(kW * 64) void scan_twopass_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) TwoPassSmem<T, FDT> sm;
  const int groups = a.D / kCh;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  // workgroup-uniform (readfirstlane keeps the bases derived from them in SGPRs)
  const int b = __builtin_amdgcn_readfirstlane(gid / groups);
  const int ch0 = __builtin_amdgcn_readfirstlane((gid % groups) * kCh);
  if (MODE != 0 && twopass_paired(a, ch0) != (MODE == 1)) return;   // the other kernel's
  twopass_body<T, K, MODE == 1, FDT>(a, sm, b, ch0);
}

template <typename T, int K, bool FDT>
hipError_t dispatch_twopass_kf(const ScanArgs &a, hipStream_t s) {
  const unsigned blocks = (unsigned)((int64_t)a.B * (a.D / kCh));
  if (a.general_a) {
    hipLaunchKernelGGL((scan_twopass_kernel<T, K, 0, FDT>), dim3(blocks), dim3(kW * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL((scan_twopass_kernel<T, K, 1, FDT>), dim3(blocks), dim3(kW * 64), 0, s, a);
    hipLaunchKernelGGL((scan_twopass_kernel<T, K, 2, FDT>), dim3(blocks), dim3(kW * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <typename T, int K>
hipError_t dispatch_twopass_k(const ScanArgs &a, hipStream_t s) {
  if (a.dtlow) {
    if constexpr (sizeof(T) == 2) return dispatch_twopass_kf<T, K, true>(a, s);
    return hipErrorInvalidValue;
  }
  return dispatch_twopass_kf<T, K, false>(a, s);
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
// chip underfilled (fewer than 2048 waves) and the sequence is long, the lane-per-state-group
// kernel runs instead.
bool use_lanes(const ScanArgs &a) {
  if (a.D % kLC != 0) return false;
  if (a.force == 1) return false;
  if (a.force == 2) return true;
  const int64_t waves = (int64_t)a.B * a.D / 64;
  return a.L > kLT && waves < 2048;
}

// d_state 16 with first-order Bbar: the two-pass kernel (its ZOH form would not fit the VGPRs:
// it keeps expm1(dt A) for the replay and needs 1 / A besides); everything else the lane kernel
template <typename T, int K>
hipError_t dispatch_few_k(const ScanArgs &a, hipStream_t s) {
  return a.N == kN && !a.zoh ? dispatch_twopass_k<T, K>(a, s) : dispatch_lanes_k<T, K>(a, s);
}

template <typename T>
hipError_t dispatch(const ScanArgs &a, hipStream_t s) {
  const bool few = use_lanes(a);
  // d_state 8, 32, 64 run on the lane kernel only (csrc/scan_n.hip otherwise)
  if (a.N != kN && !few) return hipErrorInvalidValue;
  switch (a.K) {
    case 2: return few ? dispatch_few_k<T, 2>(a, s) : dispatch_k<T, 2>(a, s);
    case 3: return few ? dispatch_few_k<T, 3>(a, s) : dispatch_k<T, 3>(a, s);
    case 4: return few ? dispatch_few_k<T, 4>(a, s) : dispatch_k<T, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan(mm_dtype dt, const ScanArgs &a, hipStream_t s) {
  if (a.N != 8 && a.N != 16 && a.N != 32 && a.N != 64) return hipErrorInvalidValue;
  if (a.dtlow && (dt != MM_BF16 || !scan_fused_dt_used(a.B, a.L, a.D, a.N, kFR, a.force, a.zoh) ||
                  !a.dtlow_lo || !a.dt_w || !a.dt_b))
    return hipErrorInvalidValue;
  return dt == MM_BF16 ? dispatch<bf16_t>(a, s) : dispatch<float>(a, s);
}

bool scan_tuned_used(int B, int L, int D, int N, uint32_t force) {
  if (N != 8 && N != 32 && N != 64) return false;
  ScanArgs a{};
  a.force = force;
  a.B = B; a.L = L; a.D = D; a.N = N;
  return use_lanes(a);
}

bool scan_fused_dt_used(int B, int L, int D, int N, int R, uint32_t force, int zoh) {
  ScanArgs a{};
  a.force = force;
  a.B = B; a.L = L; a.D = D; a.N = N;
  // the two-pass kernel (dispatch_few_k) at dt_rank 256
  return N == kN && !zoh && R == kFR && use_lanes(a);
}

}  // namespace mm
