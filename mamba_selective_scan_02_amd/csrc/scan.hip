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
// kW * kS = 128 tokens. Per block:
//  0. The block's x (with the 3 conv-window rows before it), z, dt and B|C rows were loaded
//     into LDS with direct-to-LDS 16-byte loads while the previous block was computed.
//  1. Prep (all 512 threads, one (channel, 8 tokens) run each): u = SiLU(conv1d(x) + b),
//     dt, dt*u, D*u and SiLU(z), once per (token, channel), into LDS.
//  2. Local pass: wave w takes tokens 16w .. 16w+15; lane l works on channel l/2 and states
//     8*(l%2) .. +7. The segment is scanned from h = 0, keeping exp(dt*A) of every
//     (token, state) in VGPRs (one exp per element, as in the sequential recurrence).
//  3. Compose: the segment's transfer h -> P h + S (P = exp(A * sum dt), S = the local end
//     state) goes to LDS. Thread i then owns one (channel, state) chain: it applies the 8
//     transfers in order to the block's carry-in with the page's associative operator
//     ("Parallel training via the parallel scan": (a, b) then (c, d) gives (ac, ad + b) for
//     h -> a h + b), writing each segment's h_in over that segment's P, and keeps the result
//     as the next block's carry-in.
//  4. Replay from the true h_in with the stored exp(dt*A); y_t = C_t . h_t; the two half-sums
//     of a channel meet by a DPP lane swap; y = (y_ssm + D u) * SiLU(z) goes out as bf16/f32.
constexpr int kCh = 32, kW = 8, kS = 16, kG = 8, kBlk = kW * kS;
constexpr int kHalo = 3;                  // x rows before the block (conv window, K - 1 <= 3)
constexpr int kXRows = kBlk + 16;         // staged x rows: halo + block, padded to 16-row loads

// One direct-to-LDS 16-byte load per lane: lane i of the wave fills bytes [16 i, 16 i + 16)
// of the 1 KB LDS window at `lds` (wave-uniform). Issued opaquely (see dma16_opaque): the block
// loop waits for it explicitly.
__device__ __forceinline__ void load_lds16(const void *src, void *lds) {
  dma16_opaque(src, lds_addr(lds));
}

template <typename T, bool ZOH, int K>
__global__ __launch_bounds__(kW * 64) void scan_chunked_kernel(ScanArgs a) {
  typedef typename Delta<T>::type DT;
  constexpr int xper = 16 / sizeof(T);                 // x/z elements per 16-byte chunk
  constexpr int xrow_chunks = kCh * sizeof(T) / 16;    // 16-byte chunks per staged x/z row
  constexpr int drow_chunks = kCh * sizeof(DT) / 16;
  // bf16 I/O stages x, z and dt through LDS too; fp32 I/O (small problems) reads them from
  // global memory in the prep phase, which keeps its LDS within 160 KB.
  constexpr bool kStageXZD = sizeof(T) == 2;
  constexpr int kXR = kStageXZD ? kXRows : 1, kZR = kStageXZD ? kBlk : 1;
  // staging (written by async loads); B|C double-buffered in two arrays so that the compiler
  // can tell the prefetch target from the tile being read
  __shared__ __attribute__((aligned(16))) float bc_s0[kBlk][2 * kN];
  __shared__ __attribute__((aligned(16))) float bc_s1[kBlk][2 * kN];
  __shared__ __attribute__((aligned(16))) T x_s[kXR][kCh];
  __shared__ __attribute__((aligned(16))) T z_s[kZR][kCh];
  __shared__ __attribute__((aligned(16))) DT d_s[kZR][kCh];
  // prep outputs: (dt, dt*u) and (D*u, SiLU(z)) per (token, channel); rows padded by one
  // element so that rows 1 and 8 apart fall in different LDS banks
  __shared__ __attribute__((aligned(16))) float2 pd_s[kBlk][kCh + 1];
  __shared__ __attribute__((aligned(16))) float2 eg_s[kBlk][kCh + 1];
  // segment transfers, lane-contiguous 16-byte slots: [wave][P0..3, P4..7, S0..3, S4..7][lane]
  __shared__ __attribute__((aligned(16))) float4 agg_s[kW][4][64];

  const int groups = a.D / kCh;
  const int gid = xcd_remap(blockIdx.x, gridDim.x);
  const int b = gid / groups;
  const int ch0 = (gid % groups) * kCh;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int c = lane >> 1, p = lane & 1;
  const int ch = ch0 + c;

  float A2[kG], Av[kG], iA[kG];
#pragma unroll
  for (int j = 0; j < kG; ++j) {
    Av[j] = a.A[(int64_t)ch * kN + kG * p + j];
    A2[j] = Av[j] * kLog2e;
    iA[j] = 1.0f / Av[j];
  }
  // chain thread tid <-> publishing lane ql = (tid >> 2) & 63 (channel ql/2, state half ql&1),
  // state j = 4 (tid >> 8) + (tid & 3) of that half: its P of segment w is float w*1024 + tid
  // of agg_s, its S float w*1024 + 512 + tid (conflict-free, lane-contiguous)
  const int ql = (tid >> 2) & 63, qj = 4 * (tid >> 8) + (tid & 3);
  const int64_t qidx = ((int64_t)b * a.D + ch0 + (ql >> 1)) * kN + kG * (ql & 1) + qj;
  float carry = (a.state_valid && a.state) ? a.state[qidx] : 0.f;
  // prep thread: channel pc, tokens 8*pt .. 8*pt+7 of the block
  const int pc = tid & (kCh - 1), pt = tid >> 5;
  const int pch = ch0 + pc;

  const int64_t row = 2LL * a.D;
  const T *xzb = (const T *)a.xz + (int64_t)b * a.L * row;
  const DT *db = (const DT *)a.delta + (int64_t)b * a.L * a.D;
  const float *bcb = a.bc + (int64_t)b * a.L * 2 * kN;
  T *yb = (T *)a.y + (int64_t)b * a.L * a.D;
  const int nblocks = (a.L + kBlk - 1) / kBlk;
  const int Lm1 = a.L - 1;

  // Issue the direct-to-LDS loads of block `blk` (rows past the end read row L-1 so every
  // address is valid; prep and the scan ignore those rows).
  auto stage = [&](int blk, float (*bcdst)[2 * kN]) {
    const int T0 = blk * kBlk;
    // Rows past the end read row L-1 (valid addresses; prep and the scan ignore them). Addresses
    // are a wave-uniform per-block base plus 32-bit lane offsets.
    const int rmax = Lm1 - T0;                    // last valid block-relative row
    // B|C: 128 rows x 128 B = 16 KB = 16 wave-loads; wave wv does loads wv and wv + 8
    const float *bcbase = bcb + (int64_t)T0 * 2 * kN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ld = wv + i * kW;                 // 1 KB window index
      const int r = min(ld * 8 + (lane >> 3), rmax);   // 8 lanes per 128-byte row
      load_lds16(bcbase + (uint32_t)(r * 2 * kN + (lane & 7) * 4), &bcdst[ld * 8][0]);
    }
    if (!kStageXZD) return;
    // x: kXRows rows x 64 B (bf16) = 9 wave-loads of 16 rows; row r <-> token T0 - 3 + r
    constexpr int xrpl = 64 / xrow_chunks;        // rows per wave-load
    const T *xbase = xzb + (int64_t)T0 * row + ch0;
    const uint32_t rowe = (uint32_t)row;
    for (int ld = wv; ld < kXRows / xrpl; ld += kW) {
      const int r = min(max(ld * xrpl + lane / xrow_chunks - kHalo, -T0), rmax);
      load_lds16(xbase + (int)(r * (int)rowe) + (lane % xrow_chunks) * xper, &x_s[ld * xrpl][0]);
    }
    for (int ld = wv; ld < kBlk / xrpl; ld += kW) {
      const int r = min(ld * xrpl + lane / xrow_chunks, rmax);
      load_lds16(xbase + a.D + (uint32_t)(r * rowe) + (lane % xrow_chunks) * xper,
                 &z_s[ld * xrpl][0]);
    }
    constexpr int drpl = 64 / drow_chunks;
    constexpr int dper = 16 / sizeof(DT);
    const DT *dbase = db + (int64_t)T0 * a.D + ch0;
    for (int ld = wv; ld < kBlk / drpl; ld += kW) {
      const int r = min(ld * drpl + lane / drow_chunks, rmax);
      load_lds16(dbase + (uint32_t)(r * a.D) + (lane % drow_chunks) * dper, &d_s[ld * drpl][0]);
    }
  };

  // y of block b is stored at the start of block b+1, after that block's wait, so the wait
  // for the staged tiles never has to cover freshly issued stores. Lane (c, p) owns tokens
  // tb0 + 2i + p of its wave's segment.
  float ypend[kS / 2];
  int ypend_t0 = -1;
  auto flush = [&]() {
    if (ypend_t0 < 0) return;
    // wave-uniform block base, 32-bit lane offsets (a block spans < 2^31 / sizeof(T) elements)
    T *ybase = yb + (int64_t)ypend_t0 * a.D;
    const int tl0 = wv * kS + p;
    if (ypend_t0 + kBlk <= a.L) {
#pragma unroll
      for (int i = 0; i < kS / 2; ++i)
        io<T>::st(ybase + (uint32_t)((tl0 + 2 * i) * a.D + ch), ypend[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kS / 2; ++i)
        if (ypend_t0 + tl0 + 2 * i < a.L)
          io<T>::st(ybase + (uint32_t)((tl0 + 2 * i) * a.D + ch), ypend[i]);
    }
  };
  auto block = [&](int blk, float (*bc_cur)[2 * kN], float (*bc_nxt)[2 * kN]) {
    const int T0 = blk * kBlk;
    wait_vmem_all();   // this wave's staged tiles (and its older stores) have landed
    lds_barrier();     // ... and every wave's; the previous block is fully consumed
    flush();

    // ---- 1. prep: conv + SiLU, dt, dt*u, D*u, SiLU(z) for (pc, tokens 8pt..8pt+7)
    {
      // per-channel constants, reloaded each block (cache hits) to keep them out of the
      // registers that live across the scan
      float wc[K];
#pragma unroll
      for (int k = 0; k < K; ++k) wc[k] = io<T>::cvt(((const T *)a.conv_w)[(int64_t)pch * K + k]);
      const float cb = a.conv_b ? io<T>::cvt(((const T *)a.conv_b)[pch]) : 0.0f;
      const float Dp = a.Dskip[pch];
      // block-relative token tb (tb >= -3, T0 + tb < L where it matters)
      auto getx = [&](int tb) -> float {
        if (kStageXZD) return io<T>::cvt(x_s[(kStageXZD ? tb + kHalo : 0)][pc]);
        return io<T>::cvt(xzb[(int64_t)min(T0 + tb, Lm1) * row + pch]);
      };
      auto getz = [&](int tb) -> float {
        if (kStageXZD) return io<T>::cvt(z_s[(kStageXZD ? tb : 0)][pc]);
        return io<T>::cvt(xzb[(int64_t)min(T0 + tb, Lm1) * row + a.D + pch]);
      };
      auto getd = [&](int tb) -> float {
        if (kStageXZD) return (float)d_s[(kStageXZD ? tb : 0)][pc];
        return (float)db[(int64_t)min(T0 + tb, Lm1) * a.D + pch];
      };
      float win[K - 1];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const int tb = pt * 8 - (K - 1) + j;      // block-relative token of this window row
        const int t = T0 + tb;
        float v = 0.f;
        if (t >= 0) {
          v = getx(tb);
        } else if (a.conv_valid && a.conv_state) {
          v = io<T>::cvt(((const T *)a.conv_state)[((int64_t)b * a.D + pch) * (K - 1) + (K - 1) + t]);
        }
        win[j] = v;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tb = pt * 8 + e;
        const bool valid = T0 + tb < a.L;
        const float x = getx(tb);
        float acc = cb;
#pragma unroll
        for (int j = 0; j < K - 1; ++j) acc = __builtin_fmaf(wc[j], win[j], acc);
        acc = __builtin_fmaf(wc[K - 1], x, acc);
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
        win[K - 2] = x;
        const float u = silu_f(acc);
        const float dt = valid ? getd(tb) : 0.f;
        const float z = getz(tb);
        // ZOH replays Bbar u = expm1(dt A)/A * B * u, so it keeps u where Euler keeps dt*u
        pd_s[tb][pc] = make_float2(dt, valid ? (ZOH ? u : dt * u) : 0.f);
        eg_s[tb][pc] = make_float2(valid ? Dp * u : 0.f, valid ? silu_f(z) : 0.f);
      }
    }
    lds_barrier();
    // next block's staging overlaps this block's scan (x, z, dt tiles are free after prep;
    // B|C is double-buffered)
    if (blk + 1 < nblocks) stage(blk + 1, bc_nxt);

    // ---- 2. local pass over this wave's segment
    const int tb0 = wv * kS;
    float dA[kS][kG];
    float hl[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) hl[j] = 0.f;
    float sumdt = 0.f;
#pragma unroll
    for (int t = 0; t < kS; ++t) {
      const int tb = tb0 + t;
      const float2 pd = pd_s[tb][c];
      const float dt = pd.x, du = pd.y;
      sumdt += dt;
      const float4 B0 = *(const float4 *)&bc_cur[tb][kG * p];
      const float4 B1 = *(const float4 *)&bc_cur[tb][kG * p + 4];
      const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        if (ZOH) {
          const float em1 = expm1_f(dt * Av[j]);
          dA[t][j] = em1;  // ZOH keeps expm1(dt A); exp(dt A) = 1 + it
          hl[j] = __builtin_fmaf(em1 + 1.0f, hl[j], em1 * iA[j] * Bv[j] * du);
        } else {
          dA[t][j] = exp2_hw(dt * A2[j]);
          hl[j] = __builtin_fmaf(dA[t][j], hl[j], du * Bv[j]);
        }
      }
    }
    // ---- 3. publish this segment's transfer, then compose
    {
      float P[kG];
#pragma unroll
      for (int j = 0; j < kG; ++j) P[j] = exp2_hw(A2[j] * sumdt);
      agg_s[wv][0][lane] = make_float4(P[0], P[1], P[2], P[3]);
      agg_s[wv][1][lane] = make_float4(P[4], P[5], P[6], P[7]);
      agg_s[wv][2][lane] = make_float4(hl[0], hl[1], hl[2], hl[3]);
      agg_s[wv][3][lane] = make_float4(hl[4], hl[5], hl[6], hl[7]);
    }
    lds_barrier();
    // chain pass: P of segment w becomes that segment's h_in
    {
      float *agg = &agg_s[0][0][0].x;
      float Pw[kW], Sw[kW];
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) {
        Pw[w2] = agg[w2 * 1024 + tid];
        Sw[w2] = agg[w2 * 1024 + 512 + tid];
      }
#pragma unroll
      for (int w2 = 0; w2 < kW; ++w2) {
        agg[w2 * 1024 + tid] = carry;
        carry = __builtin_fmaf(Pw[w2], carry, Sw[w2]);
      }
    }
    lds_barrier();
    float hin[kG];
    {
      const float4 H0 = agg_s[wv][0][lane], H1 = agg_s[wv][1][lane];
      hin[0] = H0.x; hin[1] = H0.y; hin[2] = H0.z; hin[3] = H0.w;
      hin[4] = H1.x; hin[5] = H1.y; hin[6] = H1.z; hin[7] = H1.w;
    }
    // ---- 4. replay from the true h_in; y from the two half-sums of the channel
    float h[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) h[j] = hin[j];
#pragma unroll
    for (int t = 0; t < kS; t += 2) {
      float ys[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tb = tb0 + t + e;
        const float4 B0 = *(const float4 *)&bc_cur[tb][kG * p];
        const float4 B1 = *(const float4 *)&bc_cur[tb][kG * p + 4];
        const float4 C0 = *(const float4 *)&bc_cur[tb][kN + kG * p];
        const float4 C1 = *(const float4 *)&bc_cur[tb][kN + kG * p + 4];
        const float Bv[kG] = {B0.x, B0.y, B0.z, B0.w, B1.x, B1.y, B1.z, B1.w};
        const float Cv[kG] = {C0.x, C0.y, C0.z, C0.w, C1.x, C1.y, C1.z, C1.w};
        const float du = pd_s[tb][c].y;
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
      const float2 eg = eg_s[tb][c];
      ypend[t / 2] = (keep + other + eg.x) * eg.y;
    }
    ypend_t0 = T0;
  };

  stage(0, bc_s0);
  for (int blk = 0; blk < nblocks; ++blk) {
    const bool odd = blk & 1;
    block(blk, odd ? bc_s1 : bc_s0, odd ? bc_s0 : bc_s1);
  }
  flush();
  if (a.state) a.state[qidx] = carry;
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
