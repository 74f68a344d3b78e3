// Host-side launchers of the mixer's kernels (internal; the ABI is include/mamba_mixer.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mamba_mixer.h"

namespace mm {

struct ConvArgs {
  const void *xz;       // [B, L, 2D]; x = first D columns
  void *u;              // [B, L, D]: fp32 u (fp32 mode) or its bf16 high part (bf16 mode)
  void *u_lo;           // [B, L, D]: bf16 mode only, bf16(u - high part)
  const void *w;        // [D, K]
  const void *bias;     // [D] or null
  const void *state;    // [B, D, K-1] or null
  int state_valid;
  int B, L, D, K;
};
hipError_t launch_conv_silu(mm_dtype dt, const ConvArgs &a, hipStream_t s);
// Rewrites state[b, i, :] with the last K-1 inputs; runs after every kernel that reads it.
hipError_t launch_conv_state_update(mm_dtype dt, const ConvArgs &a, void *state_out, hipStream_t s);

// xdbl[T, Nx] (fp32) = u[T, D] . W[Nx, D]^T. bf16 mode: u = u_hi + u_lo, two MFMA passes.
hipError_t launch_xproj(mm_dtype dt, const void *u, const void *u_lo, const void *w, float *xdbl,
                        int T, int D, int Nx, hipStream_t s);

// Per token: dt_low = RMSNorm(xdbl[:, :R]) -> dtlow [T, R] (fp32 mode: fp32; bf16 mode: bf16
// high part in dtlow, bf16 low part in dtlow_lo); B, C = RMSNorm of the next two N-slices ->
// bc [T, 2N] (fp32).
hipError_t launch_norm(mm_dtype dt, const float *xdbl, void *dtlow, void *dtlow_lo, float *bc,
                       const float *g_dt, const float *g_B, const float *g_C, int T, int R, int N,
                       float eps, hipStream_t s);

// dt[T, D] = softplus(dtlow[T, R] . Wdt[D, R]^T + bias); fp32 out
// (bf16 mode, where dtlow = hi + lo takes two MFMA passes).
hipError_t launch_dtproj(mm_dtype dt, const void *dtlow, const void *dtlow_lo, const void *w,
                         const float *bias, void *dtout, int T, int D, int R, hipStream_t s);

// bf16 I/O fused path: conv1d + SiLU -> x_proj -> RMSNorm of dt_low / B / C in one kernel.
struct XprojFusedArgs {
  const uint16_t *xz;          // [B, L, 2D] bf16
  const uint16_t *conv_w;      // [D, K] bf16
  const uint16_t *conv_b;      // [D] bf16 or null
  const uint16_t *conv_state;  // [B, D, K-1] bf16 or null
  int conv_valid;
  const uint16_t *w;           // x_proj weight [R + 2N, D] bf16
  uint16_t *dtlow, *dtlow_lo;  // [T, R] bf16 high and low parts of RMSNorm(dt_low)
  float *bc;                   // [T, 2N] RMSNorm(B) | RMSNorm(C)
  const float *g_dt, *g_B, *g_C;
  float eps;
  int B, L, D, R, K;
  int N = 16;                  // d_state: 8, 16 or 32
};
bool xproj_fused_supported(int R, int N, int D, int K);
hipError_t launch_xproj_fused(const XprojFusedArgs &a, hipStream_t s);

// bf16 I/O dt_proj: dt[T, D] (fp32) = softplus((dtlow + dtlow_lo)[T, R] . Wdt[D, R]^T + bias)
struct DtprojArgs {
  const uint16_t *dtlow, *dtlow_lo;  // [T, R] bf16
  const uint16_t *w;                 // [D, R] bf16
  const float *bias;                 // [D]
  float *dt;                         // [T, D]
  int T, D, R;
};
bool dtproj_supported(int R, int D);
hipError_t launch_dtproj_tiled(const DtprojArgs &a, hipStream_t s);

// bf16 decode step (L = 1 per sequence): partial x_proj over channel ranges, reduction +
// RMSNorm, and the fused conv / state-update / gate / conv-state kernel.
struct DecodeXprojArgs {
  const uint16_t *xz;          // [B, 2D]
  const uint16_t *conv_w;      // [D, 4]
  const uint16_t *conv_b;      // [D] or null
  const uint16_t *conv_state;  // [B, D, 3] (read; updated later by the update kernel)
  const uint16_t *w;           // [R + 32, D]
  float *part;                 // [ranges, B, R + 32]
  int B, D, R;
  int range_ch;                // channels per range (multiple of 64)
};
struct DecodeNormArgs {
  const float *part;
  int nranges;
  uint16_t *dtlow, *dtlow_lo;  // [B, R]
  float *bc;                   // [B, 32]
  const float *g_dt, *g_B, *g_C;
  float eps;
  int B, R;
};
struct DecodeUpdateArgs {
  const uint16_t *xz;          // [B, 2D]
  const uint16_t *conv_w, *conv_b;
  uint16_t *conv_state;        // [B, D, 3] in/out
  const float *dt;             // [B, D]
  const float *bc;             // [B, 32]
  const float *A, *Dskip;
  float *state;                // [B, D, 16] in/out
  uint16_t *y;                 // [B, D]
  int B, D;
};
bool decode_fast_supported(int R, int N, int D, int K);
hipError_t launch_decode_xproj(const DecodeXprojArgs &a, hipStream_t s);
hipError_t launch_decode_norm(const DecodeNormArgs &a, hipStream_t s);
hipError_t launch_decode_update(const DecodeUpdateArgs &a, bool zoh, hipStream_t s);

// C[M, N] = A[M, K] . B[N, K]^T (+ R), bf16, fp32 accumulate (row-major, lda = ldb = K)
struct GemmArgs {
  const uint16_t *A, *B;
  const uint16_t *R;           // residual [M, ldr] added to C, or null
  uint16_t *C;
  int M, N, K, ldc, ldr;
};
bool gemm_nt_supported(int M, int N, int K);
// tile: 256 or 128 (the workgroup tile); 0 picks 256 when N % 256 == 0 and the 256 x 256 tiles
// number at least 256, else 128.
hipError_t launch_gemm_nt(const GemmArgs &g, hipStream_t s, int tile = 0);
hipError_t launch_rmsnorm_rows(const uint16_t *x, const float *gamma, uint16_t *y, int T, int Dm,
                               float eps, hipStream_t s);


// ---- backward of the prefill (backward.hip). fp32 workspace arrays; T = batch * seqlen.
struct BwArgs {
  // forward inputs (io dtype unless noted) and dy
  const void *xz, *dy, *conv_w, *conv_b, *conv_state;
  int cs_valid;
  const float *ssm_state;
  int ss_valid;
  const void *x_proj_w, *dt_proj_w;
  const float *dt_b, *A, *Dskip, *g_dt, *g_B, *g_C;
  float eps;
  int zoh;
  int B, L, D, K, R, nr;   // nr = ranges per sequence
  int64_t T;
  // workspace
  float *wx32, *wdt32;     // weights in fp32 (bf16 I/O)
  float *u, *xd, *dtn, *bc;                 // [T, D], [T, R+32], [T, R], [T, 32]
  float *dt, *sig, *du;                     // [T, D]: dt holds dt_proj's product (before the
                                            // bias); the reverse scan writes d(dt_proj
                                            // pre-activation) into sig, and du
  float *rP, *rS, *rR, *dA_part;            // [B, nr, D, 16]
  float *dD_part;                           // [B, nr, D]
  float *bc_part, *dbc;                     // [T, D/32, 32], [T, 32]
  float *ddtn, *dxd, *gc;                   // [T, R], [T, R+32], [T, R+32]
  float *conv_part;                         // [B, conv strips, D, 5]
  float *conv_sum;                          // [D, 5]
  uint16_t *u_hi, *u_lo, *dp_hi, *dp_lo;    // optional bf16 hi / lo planes [T, D] of u and of
                                            // d(dt_proj pre-activation) (split products)
  // outputs
  void *dxz;
  float *d_conv_w, *d_conv_b, *d_ssm_state, *d_conv_state;
};
// stage: 0 u; 2 range transfers + carries + reverse scan + dB|dC + dz + d(dt_proj pre-act.);
// 3 RMSNorm backward; 5 conv + SiLU backward (dx, partials); 6 weights to fp32; 7 conv
// weight gradients from the column sums of the partials
hipError_t launch_backward_stage(mm_dtype dt, const BwArgs &a, int stage, hipStream_t s);
int bw_ranges(int L);
int bw_conv_strips(int L);
int64_t bw_colsum_blocks(int64_t rows);

// C[m scm + n scn] (+)= sum_k A[m sam + k sak] B[k sbk + n sbn], fp32 (16x16x4 fp32 MFMA)
// With part != null the K range may be split over up to kMaxSplit workgroups per tile (for
// short-and-wide products whose K is long); part then holds kMaxSplit * M * N floats and the
// splits are summed in a fixed order.
constexpr int kMaxSplit = 8;
struct GemmF32Args {
  const float *A, *B;
  float *C;
  int M, N, K;
  int64_t sam, sak, sbk, sbn, scm, scn;
  int accumulate;
  float *part = nullptr;
  int split = 1;
};
hipError_t launch_gemm_f32(const GemmF32Args &g, hipStream_t s);
// out[c] = sum over rows of in[rows, cols] (fixed order); part >= bw_colsum_blocks(rows) * cols
hipError_t launch_colsum(const float *in, int64_t rows, int64_t cols, float *part, float *out,
                         hipStream_t s);

// ---- split-precision bf16 products of the backward (bwgemm.hip)
// C[M, N] (+)= sum over segments s < nseg of A[s][M, K] . B[s][N, K]^T: bf16 planes whose rows
// are contiguous along K (row strides lda, ldb), fp32 out (row stride ldc). K % 64 == 0,
// N % 4 == 0; M and N otherwise arbitrary. With part != null a long K is split over up to
// kSpMaxSplit workgroups per tile; part then holds kSpMaxSplit * M * N floats and the splits
// are added in a fixed order.
constexpr int kSpMaxSplit = 32;
struct SpGemmArgs {
  const uint16_t *A[3], *B[3];
  int nseg;
  float *C;
  int M, N, K;
  int lda, ldb, ldc;
  int accumulate;
  float *part;
  int split;
};
hipError_t launch_gemm_sp(const SpGemmArgs &g, hipStream_t s);
int gemm_sp_split(int M, int N, int K);
// fp32 src[rows, cols] (row stride lds) -> bf16 hi = bf16(v), lo = bf16(v - hi) planes
// [rows, ldd], zero past cols; lo may be null (exactly-bf16 sources)
hipError_t launch_split_bf16(const float *src, int64_t rows, int cols, int64_t lds, uint16_t *hi,
                             uint16_t *lo, int ldd, hipStream_t s);
// the same split, transposed: planes [cols, ldd] with element [c][r] = src[r][c], zero for
// r >= rows; ldd % 64 == 0
hipError_t launch_tsplit_bf16(const float *src, int rows, int cols, int64_t lds, uint16_t *hi,
                              uint16_t *lo, int64_t ldd, hipStream_t s);

struct ScanArgs {
  const void *xz;       // [B, L, 2D]; x = first D columns (conv input), z = last D (gate)
  const void *conv_w;   // [D, K] io dtype
  const void *conv_b;   // [D] io dtype or null
  const void *conv_state;  // [B, D, K-1] io dtype or null (read before it is updated)
  int conv_valid;
  int K;
  const float *delta;   // [B, L, D] fp32
  const float *bc;      // [B*L, 2N]: B then C per token
  const float *A;       // [D, N]
  const float *Dskip;   // [D]
  void *y;              // [B, L, D]
  float *state;         // [B, D, N] or null
  int state_valid;
  int zoh;
  int force;            // 0: pick by size; 1: one lane per channel (d_state 16) or the general
                        // time-parallel scan; 2: lanes over (channel, state group)
  int general_a;        // 1: evaluate every exp(dt A) directly (no paired-decay shortcut)
  int B, L, D, N;
  // d_state != 16 (scan_n.hip): u from the conv kernel (fp32, or bf16 high + low parts) and
  // the per-range transfers [B, ranges, D, N] (P, and S / the range start states)
  const void *u = nullptr, *u_lo = nullptr;
  float *gP = nullptr, *gS = nullptr;
  // fused dt_proj (bf16 on the two-pass scan, dt_rank 256; scan_fused_dt_used): dt is formed in
  // the scan from the normalised dt_low planes [B*L, 256] bf16 (high, low), W_dt [D, 256] bf16
  // and the bias [D]; delta is then not read. Null dtlow: dt comes from delta.
  const uint16_t *dtlow = nullptr, *dtlow_lo = nullptr, *dt_w = nullptr;
  const float *dt_b = nullptr;
};
// N = 16; N = 8, 32, 64 when scan_tuned_used
hipError_t launch_scan(mm_dtype dt, const ScanArgs &a, hipStream_t s);
bool scan_tuned_used(int B, int L, int D, int N, uint32_t force);
// the shapes on which launch_scan accepts ScanArgs::dtlow (bf16 I/O is the caller's check)
bool scan_fused_dt_used(int B, int L, int D, int N, int R, uint32_t force, int zoh);
bool scan_n_supported(int N);
int scan_n_ranges(int L);
hipError_t launch_scan_n(mm_dtype dt, const ScanArgs &a, hipStream_t s);

}  // namespace mm
