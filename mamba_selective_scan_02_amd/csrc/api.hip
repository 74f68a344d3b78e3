// C ABI of the mixer library: argument validation, workspace layout, stage sequencing and
// the per-stage timer. Declarations and contracts: include/mamba_mixer.h.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace {

using namespace mm;

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline size_t esz(mm_dtype d) { return d == MM_BF16 ? 2 : 4; }

struct Workspace {
  bool fused_xproj;  // bf16: conv + x_proj + RMSNorm in one kernel (no u / xdbl buffers)
  bool tiled_dtproj; // bf16: token-stationary dt_proj kernel
  bool fast_decode;  // bf16 decode step: range-split x_proj, fused update (no u / xdbl buffers)
  bool scan_tuned;   // d_state 8 / 32 / 64 on the lane-per-state-group scan kernel
  bool fused_dt;     // bf16: dt_proj + softplus inside the two-pass scan (no dt buffer)
  int dec_ranges, dec_range_ch;
  size_t u, u_lo, xdbl, part, dtlow, dtlow_lo, bc, dt, gP, gS, total;
};

// the scan-selection flags as ScanArgs::force (0 by size, 1 sequential / general, 2 chunked)
uint32_t scan_force(uint32_t flags) {
  return (flags & MM_FLAG_SCAN_SEQUENTIAL) ? 1u : (flags & MM_FLAG_SCAN_CHUNKED) ? 2u : 0u;
}

// Byte offsets of the prefill intermediates for T = batch * seqlen tokens.
//   fp32 mode: u [T,D] f32 | xdbl [T,R+2N] f32 | dt_low [T,R] f32 | B,C [T,2N] f32 | dt [T,D] f32
//   bf16 mode: (u_hi, u_lo [T,D] bf16 | xdbl f32, unless fused) | dt_low hi, lo [T,R] bf16 |
//              B,C [T,2N] f32 | dt [T,D] f32 (none with the fused dt_proj)
//   bf16 decode step: partial x_proj sums [ranges, B, R+2N] f32 replace u and xdbl.
//   d_state != 16 off the lane-per-state-group scan: the general scan's per-range transfers
//   P, S [B, ranges, D, N] f32.
Workspace layout(const mm_shape &s, bool decode) {
  const size_t T = (size_t)s.batch * s.seqlen;
  const bool bf = s.io_dtype == MM_BF16;
  const size_t e = esz(s.io_dtype);
  Workspace w;
  // d_state 8 / 32 / 64 on the lane-per-state-group kernel (which recomputes u from x)
  w.scan_tuned = !decode && scan_tuned_used(s.batch, s.seqlen, s.d_inner, s.d_state,
                                            scan_force(s.flags));
  // one workgroup per 128 tokens: worth it once there are enough tokens to fill the chip; it
  // writes no u, so d_state != 16 takes it only where the scan recomputes u
  w.fused_xproj = !decode && bf && T >= 32768 &&
                  xproj_fused_supported(s.dt_rank, s.d_state, s.d_inner, s.d_conv) &&
                  (s.d_state == 16 || w.scan_tuned);
  w.tiled_dtproj = bf && dtproj_supported(s.dt_rank, s.d_inner);
  w.fused_dt = !decode && bf && (s.flags & MM_FLAG_FUSED_DTPROJ) &&
               scan_fused_dt_used(s.batch, s.seqlen, s.d_inner, s.d_state, s.dt_rank,
                                  scan_force(s.flags), (s.flags & MM_FLAG_ZOH_B) ? 1 : 0);
  w.fast_decode = decode && bf && decode_fast_supported(s.dt_rank, s.d_state, s.d_inner, s.d_conv);
  w.dec_ranges = 0;
  w.dec_range_ch = 0;
  if (w.fast_decode) {
    // enough (sequence tile, channel range) workgroups to fill the chip
    const int seq_tiles = (s.batch + 63) / 64;
    const int chunks = s.d_inner / 64;
    const int want = std::min(chunks, std::max(1, (256 + seq_tiles - 1) / seq_tiles));
    w.dec_range_ch = (chunks + want - 1) / want * 64;
    w.dec_ranges = (s.d_inner + w.dec_range_ch - 1) / w.dec_range_ch;
  }
  const bool no_u = w.fused_xproj || w.fast_decode;
  size_t o = 0;
  w.u = o; if (!no_u) o += up(T * s.d_inner * e);
  w.u_lo = o; if (bf && !no_u) o += up(T * s.d_inner * 2);
  w.xdbl = o; if (!no_u) o += up(T * (s.dt_rank + 2 * s.d_state) * 4);
  w.part = o; if (w.fast_decode) o += up((size_t)w.dec_ranges * T * (s.dt_rank + 2 * s.d_state) * 4);
  w.dtlow = o; o += up(T * s.dt_rank * e);
  w.dtlow_lo = o; if (bf) o += up(T * s.dt_rank * 2);
  w.bc = o; o += up(T * 2 * s.d_state * 4);
  w.dt = o; if (!w.fused_dt) o += up(T * s.d_inner * 4);
  // d_state != 16 off the lane kernel: per-range transfers of the general scan
  const size_t gsz = s.d_state != 16 && !w.scan_tuned
                         ? (size_t)s.batch * scan_n_ranges(s.seqlen) * s.d_inner * s.d_state * 4 : 0;
  w.gP = o; o += up(gsz);
  w.gS = o; o += up(gsz);
  w.total = o;
  return w;
}

bool aligned(const void *p) { return ((uintptr_t)p & 15) == 0; }

mm_status check_shape(const mm_shape *s, bool decode) {
  if (!s) return MM_ERR_INVALID_ARG;
  if (s->batch <= 0 || s->seqlen <= 0 || s->d_inner <= 0 || s->d_state <= 0 || s->d_conv <= 0 ||
      s->dt_rank <= 0 || !(s->rms_eps > 0.0f))
    return MM_ERR_INVALID_ARG;
  {  // the dtype arrives from C as any int: read its bytes as an int before using the enum
    int dt = 0;
    std::memcpy(&dt, &s->io_dtype, sizeof(dt));
    if (dt != MM_F32 && dt != MM_BF16) return MM_ERR_INVALID_ARG;
  }
  if (s->flags & ~(uint32_t)(MM_FLAG_ZOH_B | MM_FLAG_SCAN_SEQUENTIAL | MM_FLAG_SCAN_CHUNKED |
                             MM_FLAG_SCAN_GENERAL_A | MM_FLAG_FUSED_DTPROJ))
    return MM_ERR_INVALID_ARG;
  if ((s->flags & MM_FLAG_SCAN_SEQUENTIAL) && (s->flags & MM_FLAG_SCAN_CHUNKED))
    return MM_ERR_INVALID_ARG;
  if (decode && s->seqlen != 1) return MM_ERR_INVALID_ARG;
  if ((s->d_state != 16 && !scan_n_supported(s->d_state)) || s->d_conv < 2 || s->d_conv > 4 ||
      s->d_inner % 64 != 0)
    return MM_ERR_UNSUPPORTED;
  if (s->io_dtype == MM_BF16 && (s->dt_rank % 64 != 0 || s->d_inner % 128 != 0))
    return MM_ERR_UNSUPPORTED;
  if (s->io_dtype == MM_F32 && s->dt_rank > 1024) return MM_ERR_UNSUPPORTED;
  // index arithmetic inside kernels uses 64-bit offsets, grid sizes 32-bit counts
  const double T = (double)s->batch * s->seqlen;
  if (T * s->d_inner / 8 > 2e9) return MM_ERR_UNSUPPORTED;
  return MM_OK;
}

mm_status check_params(const mm_params *p) {
  if (!p) return MM_ERR_INVALID_ARG;
  const void *req[] = {p->conv_w, p->x_proj_w, p->dt_proj_w, p->dt_proj_b, p->A,
                       p->Dskip,  p->dt_norm_w, p->B_norm_w, p->C_norm_w};
  for (const void *q : req)
    if (!q || !aligned(q)) return MM_ERR_INVALID_ARG;
  if (p->conv_b && !aligned(p->conv_b)) return MM_ERR_INVALID_ARG;
  return MM_OK;
}

}  // namespace

struct mm_stage_timer {
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> pool;
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

// Brackets one stage with a pair of events when a timer is given.
struct StageScope {
  mm_stage_timer *t;
  hipStream_t s;
  mm_stage_timer::Rec rec{};
  StageScope(mm_stage_timer *t_, hipStream_t s_, int stage) : t(t_), s(s_) {
    if (!t) return;
    rec.stage = stage;
    rec.a = t->get();
    rec.b = t->get();
    if (rec.a) (void)hipEventRecord(rec.a, s);   // timing only: a failed record drops the sample
  }
  ~StageScope() {
    if (!t || !rec.a || !rec.b) return;
    (void)hipEventRecord(rec.b, s);
    t->recs.push_back(rec);
  }
};

#define MM_TRY(expr)                                   \
  do {                                                 \
    if ((expr) != hipSuccess) return MM_ERR_HIP;       \
  } while (0)

// bf16 decode step with d_conv 4: range-split x_proj (conv recomputed per fragment) -> partial
// reduction + RMSNorm -> dt_proj -> one kernel for conv, state update, gate and conv state.
mm_status run_decode_fast(const mm_shape *s, const mm_params *p, const Workspace &w,
                          const void *xz, void *y, void *conv_state, float *ssm_state, char *ws,
                          hipStream_t st, mm_stage_timer *timer) {
  const int B = s->batch, D = s->d_inner, R = s->dt_rank;
  float *part = (float *)(ws + w.part);
  uint16_t *dtlow = (uint16_t *)(ws + w.dtlow), *dtlow_lo = (uint16_t *)(ws + w.dtlow_lo);
  float *bc = (float *)(ws + w.bc);
  float *delta = (float *)(ws + w.dt);
  const uint16_t *cw = (const uint16_t *)p->conv_w, *cb = (const uint16_t *)p->conv_b;
  {
    StageScope sc(timer, st, MM_STAGE_XPROJ);
    DecodeXprojArgs xa{(const uint16_t *)xz, cw, cb, (const uint16_t *)conv_state,
                       (const uint16_t *)p->x_proj_w, part, B, D, R, w.dec_range_ch};
    MM_TRY(launch_decode_xproj(xa, st));
  }
  {
    StageScope sc(timer, st, MM_STAGE_NORM);
    DecodeNormArgs na{part, w.dec_ranges, dtlow, dtlow_lo, bc, p->dt_norm_w, p->B_norm_w,
                      p->C_norm_w, s->rms_eps, B, R};
    MM_TRY(launch_decode_norm(na, st));
  }
  {
    StageScope sc(timer, st, MM_STAGE_DTPROJ);
    if (w.tiled_dtproj) {
      DtprojArgs da{dtlow, dtlow_lo, (const uint16_t *)p->dt_proj_w, p->dt_proj_b, delta, B, D, R};
      MM_TRY(launch_dtproj_tiled(da, st));
    } else {
      MM_TRY(launch_dtproj(MM_BF16, dtlow, dtlow_lo, p->dt_proj_w, p->dt_proj_b, delta, B, D, R,
                           st));
    }
  }
  {
    StageScope sc(timer, st, MM_STAGE_SCAN);
    DecodeUpdateArgs ua{(const uint16_t *)xz, cw, cb, (uint16_t *)conv_state, delta, bc, p->A,
                        p->Dskip, ssm_state, (uint16_t *)y, B, D};
    MM_TRY(launch_decode_update(ua, (s->flags & MM_FLAG_ZOH_B) != 0, st));
  }
  return MM_OK;
}

mm_status run_mixer(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                    void *conv_state, float *ssm_state, int states_valid, void *workspace,
                    size_t workspace_bytes, hipStream_t st, mm_stage_timer *timer, bool decode) {
  const Workspace w = layout(*s, decode);
  if (w.fast_decode)
    return run_decode_fast(s, p, w, xz, y, conv_state, ssm_state, (char *)workspace, st, timer);
  char *ws = (char *)workspace;
  const int B = s->batch, L = s->seqlen, D = s->d_inner, N = s->d_state, K = s->d_conv;
  const int R = s->dt_rank, T = B * L;
  const mm_dtype dt = s->io_dtype;
  void *u = ws + w.u;
  void *u_lo = ws + w.u_lo;
  float *xdbl = (float *)(ws + w.xdbl);
  void *dtlow = ws + w.dtlow;
  void *dtlow_lo = ws + w.dtlow_lo;
  float *bc = (float *)(ws + w.bc);
  float *delta = (float *)(ws + w.dt);
  (void)workspace_bytes;
  const int conv_valid = states_valid && conv_state != nullptr;

  ConvArgs ca{xz, u, u_lo, p->conv_w, p->conv_b, conv_state, conv_valid, B, L, D, K};
  if (w.fused_xproj) {
    StageScope sc(timer, st, MM_STAGE_XPROJ);
    XprojFusedArgs xa{(const uint16_t *)xz, (const uint16_t *)p->conv_w, (const uint16_t *)p->conv_b,
                      (const uint16_t *)conv_state, conv_valid, (const uint16_t *)p->x_proj_w,
                      (uint16_t *)dtlow, (uint16_t *)dtlow_lo, bc, p->dt_norm_w, p->B_norm_w,
                      p->C_norm_w, s->rms_eps, B, L, D, R, K, N};
    MM_TRY(launch_xproj_fused(xa, st));
  } else {
    {
      StageScope sc(timer, st, MM_STAGE_CONV);
      MM_TRY(launch_conv_silu(dt, ca, st));
    }
    {
      StageScope sc(timer, st, MM_STAGE_XPROJ);
      MM_TRY(launch_xproj(dt, u, u_lo, p->x_proj_w, xdbl, T, D, R + 2 * N, st));
    }
    {
      StageScope sc(timer, st, MM_STAGE_NORM);
      MM_TRY(launch_norm(dt, xdbl, dtlow, dtlow_lo, bc, p->dt_norm_w, p->B_norm_w, p->C_norm_w, T,
                         R, N, s->rms_eps, st));
    }
  }
  if (!w.fused_dt) {
    StageScope sc(timer, st, MM_STAGE_DTPROJ);
    if (w.tiled_dtproj) {
      DtprojArgs da{(const uint16_t *)dtlow, (const uint16_t *)dtlow_lo,
                    (const uint16_t *)p->dt_proj_w, p->dt_proj_b, delta, T, D, R};
      MM_TRY(launch_dtproj_tiled(da, st));
    } else {
      MM_TRY(launch_dtproj(dt, dtlow, dtlow_lo, p->dt_proj_w, p->dt_proj_b, delta, T, D, R, st));
    }
  }
  {
    StageScope sc(timer, st, MM_STAGE_SCAN);
    ScanArgs sa{xz, p->conv_w, p->conv_b, conv_state, conv_valid, K, delta, bc, p->A, p->Dskip,
                y, ssm_state, states_valid && ssm_state != nullptr,
                (s->flags & MM_FLAG_ZOH_B) ? 1 : 0,
                (int)scan_force(s->flags), (s->flags & MM_FLAG_SCAN_GENERAL_A) ? 1 : 0,
                B, L, D, N};
    if (w.fused_dt) {
      sa.delta = nullptr;
      sa.dtlow = (const uint16_t *)dtlow;
      sa.dtlow_lo = (const uint16_t *)dtlow_lo;
      sa.dt_w = (const uint16_t *)p->dt_proj_w;
      sa.dt_b = p->dt_proj_b;
    }
    if (N == 16 || w.scan_tuned) {
      MM_TRY(launch_scan(dt, sa, st));
    } else {
      sa.u = u;
      sa.u_lo = u_lo;
      sa.gP = (float *)(ws + w.gP);
      sa.gS = (float *)(ws + w.gS);
      MM_TRY(launch_scan_n(dt, sa, st));
    }
  }
  if (conv_state) {
    // last: the conv and scan kernels above read the carried conv state
    StageScope sc(timer, st, MM_STAGE_CONV_STATE);
    MM_TRY(launch_conv_state_update(dt, ca, conv_state, st));
  }
  return MM_OK;
}

mm_status prefill_impl(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                       void *conv_state, float *ssm_state, int states_valid, void *workspace,
                       size_t workspace_bytes, void *stream, mm_stage_timer *timer) {
  mm_status r = check_shape(s, false);
  if (r != MM_OK) return r;
  if ((r = check_params(p)) != MM_OK) return r;
  if (!xz || !y || !aligned(xz) || !aligned(y) || xz == y) return MM_ERR_INVALID_ARG;
  if ((conv_state && !aligned(conv_state)) || (ssm_state && !aligned(ssm_state)))
    return MM_ERR_INVALID_ARG;
  if (states_valid != 0 && states_valid != 1) return MM_ERR_INVALID_ARG;
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) ||
      workspace_bytes < layout(*s, false).total)
    return MM_ERR_WORKSPACE;
  return run_mixer(s, p, xz, y, conv_state, ssm_state, states_valid, workspace, workspace_bytes,
                   (hipStream_t)stream, timer, false);
}

mm_status decode_impl(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                      void *conv_state, float *ssm_state, void *workspace, size_t workspace_bytes,
                      void *stream, mm_stage_timer *timer) {
  mm_status r = check_shape(s, true);
  if (r != MM_OK) return r;
  if ((r = check_params(p)) != MM_OK) return r;
  if (!xz || !y || !conv_state || !ssm_state || xz == y) return MM_ERR_INVALID_ARG;
  if (!aligned(xz) || !aligned(y) || !aligned(conv_state) || !aligned(ssm_state))
    return MM_ERR_INVALID_ARG;
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) ||
      workspace_bytes < layout(*s, true).total)
    return MM_ERR_WORKSPACE;
  return run_mixer(s, p, xz, y, conv_state, ssm_state, 1, workspace, workspace_bytes,
                   (hipStream_t)stream, timer, true);
}

// Layer workspace: x_norm [T, d_model] bf16 | xz [T, 2D] bf16 | y [T, D] bf16 | mixer workspace
struct LayerWs {
  size_t xn, xz, y, mixer, total;
};
LayerWs layer_layout(const mm_shape &s, int d_model) {
  const size_t T = (size_t)s.batch * s.seqlen;
  LayerWs w;
  size_t o = 0;
  w.xn = o; o += up(T * d_model * 2);
  w.xz = o; o += up(T * 2 * s.d_inner * 2);
  w.y = o; o += up(T * s.d_inner * 2);
  w.mixer = o; o += layout(s, false).total;
  w.total = o;
  return w;
}

mm_status check_layer(const mm_shape *s, int d_model, const mm_layer_params *p) {
  mm_status r = check_shape(s, false);
  if (r != MM_OK) return r;
  if (d_model <= 0) return MM_ERR_INVALID_ARG;
  if (s->io_dtype != MM_BF16 || d_model % 128 != 0) return MM_ERR_UNSUPPORTED;
  const int T = s->batch * s->seqlen;
  if (!gemm_nt_supported(T, 2 * s->d_inner, d_model) || !gemm_nt_supported(T, d_model, s->d_inner))
    return MM_ERR_UNSUPPORTED;
  if (!p) return MM_ERR_INVALID_ARG;
  if (!p->norm_w || !p->in_proj_w || !p->out_proj_w || !aligned(p->norm_w) ||
      !aligned(p->in_proj_w) || !aligned(p->out_proj_w) || !(p->norm_eps > 0.0f))
    return MM_ERR_INVALID_ARG;
  return check_params(&p->mixer);
}

mm_status layer_impl(const mm_shape *s, int d_model, const mm_layer_params *p, const void *x,
                     void *out, void *conv_state, float *ssm_state, int states_valid,
                     void *workspace, size_t workspace_bytes, void *stream, mm_stage_timer *timer) {
  mm_status r = check_layer(s, d_model, p);
  if (r != MM_OK) return r;
  if (!x || !out || !aligned(x) || !aligned(out) || x == out) return MM_ERR_INVALID_ARG;
  if ((conv_state && !aligned(conv_state)) || (ssm_state && !aligned(ssm_state)))
    return MM_ERR_INVALID_ARG;
  if (states_valid != 0 && states_valid != 1) return MM_ERR_INVALID_ARG;
  const LayerWs w = layer_layout(*s, d_model);
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) || workspace_bytes < w.total)
    return MM_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const int T = s->batch * s->seqlen, D = s->d_inner;
  uint16_t *xn = (uint16_t *)(ws + w.xn), *xz = (uint16_t *)(ws + w.xz), *y = (uint16_t *)(ws + w.y);
  {
    StageScope sc(timer, st, MM_STAGE_LAYER_NORM);
    MM_TRY(launch_rmsnorm_rows((const uint16_t *)x, p->norm_w, xn, T, d_model, p->norm_eps, st));
  }
  {
    StageScope sc(timer, st, MM_STAGE_IN_PROJ);
    GemmArgs g{xn, (const uint16_t *)p->in_proj_w, nullptr, xz, T, 2 * D, d_model, 2 * D, 0};
    MM_TRY(launch_gemm_nt(g, st));
  }
  r = run_mixer(s, &p->mixer, xz, y, conv_state, ssm_state, states_valid, ws + w.mixer,
                workspace_bytes - w.mixer, st, timer, false);
  if (r != MM_OK) return r;
  {
    StageScope sc(timer, st, MM_STAGE_OUT_PROJ);
    GemmArgs g{y, (const uint16_t *)p->out_proj_w, (const uint16_t *)x, (uint16_t *)out, T,
               d_model, D, d_model, d_model};
    MM_TRY(launch_gemm_nt(g, st));
  }
  return MM_OK;
}

// Backward workspace (fp32 arrays; T = batch * seqlen, W = dt_rank + 32, nr = ranges). With
// bf16 I/O the products run on split bf16 planes (bwgemm.hip): the planes of u live in du
// until the reverse scan writes du, those of u^T in dt once the scans have read it ([D, Tp],
// Tp = T rounded up to 64); d(dt_proj pre-activation) and its transpose, the narrow planes and
// the weight copies get their own regions.
struct BwWs {
  size_t wx32, wdt32, u, xd, dtn, bc, dt, sig, dpp, du, dpT, rP, rS, rR, dA_part, dD_part, bc_part,
      dbc, ddtn, dxd, gc, cs_part, gsum, conv_part, conv_sum, gemm_part;
  size_t wdtp, wdtT, wxT, dtn_s, dtnT, dxd_s, dxdT;   // bf16 planes (split products only)
  size_t total;
};
inline int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }
// the split-bf16 products serve bf16 I/O up to 4M tokens (32-bit lane offsets in a tile)
inline bool bw_split_products(const mm_shape &s) {
  return s.io_dtype == MM_BF16 && pad64((int64_t)s.batch * s.seqlen) <= (1 << 22);
}
BwWs bw_layout(const mm_shape &s) {
  const size_t T = (size_t)s.batch * s.seqlen, D = s.d_inner, R = s.dt_rank, W = R + 32;
  const size_t Tp = (size_t)pad64((int64_t)T), Rp = (size_t)pad64((int64_t)R),
               Wp = (size_t)pad64((int64_t)W);
  const bool sp = bw_split_products(s);
  const size_t nr = (size_t)bw_ranges(s.seqlen), SR = (size_t)s.batch * nr * D * 16;
  const size_t nbT = (size_t)bw_colsum_blocks((int64_t)T);
  const size_t nbR = (size_t)bw_colsum_blocks((int64_t)s.batch * nr);
  const size_t nstrip = (size_t)s.batch * bw_conv_strips(s.seqlen);
  const size_t nbS = (size_t)bw_colsum_blocks((int64_t)nstrip);
  BwWs w;
  size_t o = 0;
  auto take = [&](size_t &f, size_t floats) { f = o; o += up(floats * 4); };
  take(w.wx32, W * D);
  take(w.wdt32, D * R);
  take(w.u, T * D);
  take(w.xd, T * W);
  take(w.dtn, T * R);
  take(w.bc, T * 32);
  take(w.dt, (sp ? Tp : T) * D);
  take(w.sig, T * D);
  take(w.dpp, sp ? T * D : 0);    // bf16 hi / lo planes of dp [T, D]
  take(w.du, T * D);
  take(w.dpT, sp ? Tp * D : 0);   // bf16 hi / lo planes of dp^T [D, Tp]
  take(w.rP, SR);
  take(w.rS, SR);
  take(w.rR, SR);
  take(w.dA_part, SR);
  take(w.dD_part, (size_t)s.batch * nr * D);
  take(w.bc_part, T * (D / 32) * 32);   // per token, per 32-channel group of the reverse scan
  take(w.dbc, T * 32);
  take(w.ddtn, T * R);
  take(w.dxd, T * W);
  take(w.gc, T * W);
  take(w.cs_part, std::max(std::max(nbT * std::max(D, W), nbR * D * 16), nbS * D * 5));
  take(w.gsum, W);
  take(w.conv_part, nstrip * D * 5);
  take(w.conv_sum, D * 5);
  take(w.gemm_part, (size_t)(sp ? kSpMaxSplit : kMaxSplit) * D * std::max(W, R));
  // bf16 planes: two bf16 per float of take()
  auto planes = [&](size_t &f, size_t elems) { take(f, sp ? (elems + 1) / 2 : 0); };
  planes(w.wdtp, D * Rp);
  planes(w.wdtT, R * D);
  planes(w.wxT, D * Wp);
  planes(w.dtn_s, 2 * T * Rp);
  planes(w.dtnT, 2 * R * Tp);
  planes(w.dxd_s, 2 * T * Wp);
  planes(w.dxdT, 2 * W * Tp);
  w.total = o;
  return w;
}

mm_status check_backward(const mm_shape *s, const mm_params *p, const void *xz, const void *dy,
                         const void *conv_state, const float *ssm_state, int states_valid,
                         const mm_grads *g) {
  mm_status r = check_shape(s, false);
  if (r != MM_OK) return r;
  // the backward's lanes are (channel, 16 states)
  if (s->dt_rank > 1024 || s->d_state != 16) return MM_ERR_UNSUPPORTED;
  r = check_params(p);
  if (r != MM_OK) return r;
  if (!xz || !dy || !g || !aligned(xz) || !aligned(dy)) return MM_ERR_INVALID_ARG;
  if (states_valid != 0 && states_valid != 1) return MM_ERR_INVALID_ARG;
  if ((conv_state && !aligned(conv_state)) || (ssm_state && !aligned(ssm_state)))
    return MM_ERR_INVALID_ARG;
  const void *req[] = {g->dxz, g->conv_w, g->x_proj_w, g->dt_proj_w, g->dt_proj_b, g->A,
                       g->Dskip, g->dt_norm_w, g->B_norm_w, g->C_norm_w};
  for (const void *q : req)
    if (!q || !aligned(q)) return MM_ERR_INVALID_ARG;
  if ((p->conv_b != nullptr) != (g->conv_b != nullptr)) return MM_ERR_INVALID_ARG;
  if (g->conv_b && !aligned(g->conv_b)) return MM_ERR_INVALID_ARG;
  if ((g->conv_state && !aligned(g->conv_state)) || (g->ssm_state && !aligned(g->ssm_state)))
    return MM_ERR_INVALID_ARG;
  if (g->dxz == xz || g->dxz == dy) return MM_ERR_INVALID_ARG;
  return MM_OK;
}

mm_status backward_impl(const mm_shape *s, const mm_params *p, const void *xz, const void *dy,
                        const void *conv_state, const float *ssm_state, int states_valid,
                        const mm_grads *g, void *workspace, size_t workspace_bytes, void *stream,
                        mm_stage_timer *timer) {
  mm_status r = check_backward(s, p, xz, dy, conv_state, ssm_state, states_valid, g);
  if (r != MM_OK) return r;
  const BwWs w = bw_layout(*s);
  if (!workspace || ((uintptr_t)workspace & (kAlign - 1)) || workspace_bytes < w.total)
    return MM_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  auto F = [&](size_t off) { return (float *)(ws + off); };
  const int B = s->batch, L = s->seqlen, D = s->d_inner, R = s->dt_rank, W = R + 32;
  const int64_t T = (int64_t)B * L;
  const bool bf = s->io_dtype == MM_BF16;

  BwArgs a{};
  a.xz = xz; a.dy = dy; a.conv_w = p->conv_w; a.conv_b = p->conv_b;
  a.conv_state = conv_state; a.cs_valid = states_valid && conv_state;
  a.ssm_state = ssm_state; a.ss_valid = states_valid && ssm_state;
  a.x_proj_w = p->x_proj_w; a.dt_proj_w = p->dt_proj_w;
  a.dt_b = p->dt_proj_b; a.A = p->A; a.Dskip = p->Dskip;
  a.g_dt = p->dt_norm_w; a.g_B = p->B_norm_w; a.g_C = p->C_norm_w;
  a.eps = s->rms_eps; a.zoh = (s->flags & MM_FLAG_ZOH_B) ? 1 : 0;
  a.B = B; a.L = L; a.D = D; a.K = s->d_conv; a.R = R; a.nr = bw_ranges(L); a.T = T;
  a.wx32 = F(w.wx32); a.wdt32 = F(w.wdt32); a.u = F(w.u); a.xd = F(w.xd); a.dtn = F(w.dtn);
  a.bc = F(w.bc); a.dt = F(w.dt); a.sig = F(w.sig); a.du = F(w.du);
  a.rP = F(w.rP); a.rS = F(w.rS); a.rR = F(w.rR); a.dA_part = F(w.dA_part);
  a.dD_part = F(w.dD_part); a.bc_part = F(w.bc_part); a.dbc = F(w.dbc); a.ddtn = F(w.ddtn);
  a.dxd = F(w.dxd); a.gc = F(w.gc); a.conv_part = F(w.conv_part);
  a.conv_sum = F(w.conv_sum);
  a.dxz = g->dxz; a.d_conv_w = g->conv_w; a.d_conv_b = g->conv_b;
  a.d_ssm_state = g->ssm_state; a.d_conv_state = g->conv_state;
  const float *wx = bf ? a.wx32 : (const float *)p->x_proj_w;
  const float *wdt = bf ? a.wdt32 : (const float *)p->dt_proj_w;
  float *cs = F(w.cs_part);
  // split-bf16 planes (bf16 I/O)
  const bool sp = bw_split_products(*s);
  const int Tp = (int)pad64(T), Rp = (int)pad64(R), Wp = (int)pad64(W);
  auto H = [&](size_t off) { return (uint16_t *)(ws + off); };
  uint16_t *wdtp = H(w.wdtp), *wdtT = H(w.wdtT), *wxT = H(w.wxT);
  uint16_t *u_hi = H(w.du), *u_lo = u_hi + T * D;
  uint16_t *dtn_hi = H(w.dtn_s), *dtn_lo = dtn_hi + T * Rp;
  uint16_t *dtnT_hi = H(w.dtnT), *dtnT_lo = dtnT_hi + (int64_t)R * Tp;
  uint16_t *dp_hi = H(w.dpp), *dp_lo = dp_hi + T * D;
  uint16_t *dpT_hi = H(w.dpT), *dpT_lo = dpT_hi + (int64_t)D * Tp;
  uint16_t *dxd_hi = H(w.dxd_s), *dxd_lo = dxd_hi + T * Wp;
  uint16_t *dxdT_hi = H(w.dxdT), *dxdT_lo = dxdT_hi + (int64_t)W * Tp;
  uint16_t *uT_hi = H(w.dt), *uT_lo = uT_hi + (int64_t)D * Tp;
  if (sp) {   // the u and dp planes come from the kernels that form u and dp
    a.u_hi = u_hi; a.u_lo = u_lo;
    a.dp_hi = dp_hi; a.dp_lo = dp_lo;
  }

  {
    StageScope sc(timer, st, MM_STAGE_BWD_RECOMPUTE);
    if (bf) MM_TRY(launch_backward_stage(s->io_dtype, a, 6, st));
    if (sp) {   // exactly-bf16 weight copies: W_dt [D, Rp], W_dt^T [R, D], W_x^T [D, Wp]
      MM_TRY(launch_split_bf16(a.wdt32, D, R, R, wdtp, nullptr, Rp, st));
      MM_TRY(launch_tsplit_bf16(a.wdt32, D, R, R, wdtT, nullptr, D, st));
      MM_TRY(launch_tsplit_bf16(a.wx32, W, D, D, wxT, nullptr, Wp, st));
    }
    MM_TRY(launch_backward_stage(s->io_dtype, a, 0, st));                    // u
    if (sp) {   // xdbl = u W_x^T on the planes of u (in du, which the scan writes later)
      MM_TRY(launch_xproj(MM_BF16, u_hi, u_lo, p->x_proj_w, a.xd, (int)T, D, W, st));
    } else {
      MM_TRY(launch_gemm_f32({a.u, wx, a.xd, (int)T, W, D, D, 1, 1, D, W, 1, 0}, st));   // xdbl
    }
    MM_TRY(launch_norm(MM_F32, a.xd, a.dtn, nullptr, a.bc, a.g_dt, a.g_B, a.g_C, (int)T, R, 16,
                       a.eps, st));
    if (sp) {   // dt_proj's product on the planes of dt_low
      MM_TRY(launch_split_bf16(a.dtn, T, R, R, dtn_hi, dtn_lo, Rp, st));
      MM_TRY(launch_gemm_sp({{dtn_hi, dtn_lo, nullptr}, {wdtp, wdtp, nullptr}, 2, a.dt, (int)T, D,
                             Rp, Rp, Rp, D, 0, nullptr, 1}, st));
    } else {
      MM_TRY(launch_gemm_f32({a.dtn, wdt, a.dt, (int)T, D, R, R, 1, 1, R, D, 1, 0}, st));
    }
  }
  {
    StageScope sc(timer, st, MM_STAGE_BWD_SCAN);
    MM_TRY(launch_backward_stage(s->io_dtype, a, 2, st));
    MM_TRY(launch_colsum(a.dA_part, (int64_t)B * a.nr, (int64_t)D * 16, cs, g->A, st));
    MM_TRY(launch_colsum(a.dD_part, (int64_t)B * a.nr, D, cs, g->Dskip, st));
  }
  {
    StageScope sc(timer, st, MM_STAGE_BWD_PROJ);
    float *dp = a.sig;   // d / d (dt_proj pre-activation), [T, D]
    MM_TRY(launch_colsum(dp, T, D, cs, g->dt_proj_b, st));
    float *gp = F(w.gemm_part);
    if (sp) {
      // planes of dp^T and dt_low^T ([D | R, Tp]); those of dp are the reverse scan's
      MM_TRY(launch_tsplit_bf16(dp, (int)T, D, D, dpT_hi, dpT_lo, Tp, st));
      MM_TRY(launch_tsplit_bf16(a.dtn, (int)T, R, R, dtnT_hi, dtnT_lo, Tp, st));
      // d W_dt [D, R] = dp^T dt_low (over tokens); d dt_low [T, R] = dp W_dt
      MM_TRY(launch_gemm_sp({{dpT_hi, dpT_hi, dpT_lo}, {dtnT_hi, dtnT_lo, dtnT_hi}, 3,
                             g->dt_proj_w, D, R, Tp, Tp, Tp, R, 0, gp, 1}, st));
      MM_TRY(launch_gemm_sp({{dp_hi, dp_lo, nullptr}, {wdtT, wdtT, nullptr}, 2, a.ddtn, (int)T, R,
                             D, D, D, R, 0, nullptr, 1}, st));
    } else {
      MM_TRY(launch_gemm_f32({dp, a.dtn, g->dt_proj_w, D, R, (int)T, 1, D, R, 1, R, 1, 0, gp}, st));
      MM_TRY(launch_gemm_f32({dp, wdt, a.ddtn, (int)T, R, D, D, 1, R, 1, R, 1, 0}, st));
    }
    MM_TRY(launch_backward_stage(s->io_dtype, a, 3, st));                    // RMSNorm backward
    MM_TRY(launch_colsum(a.gc, T, W, cs, F(w.gsum), st));
    MM_TRY(hipMemcpyAsync(g->dt_norm_w, F(w.gsum), (size_t)R * 4, hipMemcpyDeviceToDevice, st));
    MM_TRY(hipMemcpyAsync(g->B_norm_w, F(w.gsum) + R, 64, hipMemcpyDeviceToDevice, st));
    MM_TRY(hipMemcpyAsync(g->C_norm_w, F(w.gsum) + R + 16, 64, hipMemcpyDeviceToDevice, st));
    if (sp) {
      // planes of dxdbl [T, Wp] and dxdbl^T [W, Tp], u^T [D, Tp] (in dt)
      MM_TRY(launch_split_bf16(a.dxd, T, W, W, dxd_hi, dxd_lo, Wp, st));
      MM_TRY(launch_tsplit_bf16(a.dxd, (int)T, W, W, dxdT_hi, dxdT_lo, Tp, st));
      MM_TRY(launch_tsplit_bf16(a.u, (int)T, D, D, uT_hi, uT_lo, Tp, st));
      // d W_x [W, D] = dxdbl^T u (over tokens); du += dxdbl W_x
      MM_TRY(launch_gemm_sp({{dxdT_hi, dxdT_hi, dxdT_lo}, {uT_hi, uT_lo, uT_hi}, 3, g->x_proj_w,
                             W, D, Tp, Tp, Tp, D, 0, gp, 1}, st));
      MM_TRY(launch_gemm_sp({{dxd_hi, dxd_lo, nullptr}, {wxT, wxT, nullptr}, 2, a.du, (int)T, D,
                             Wp, Wp, Wp, D, 1, nullptr, 1}, st));
    } else {
      // d x_proj_w [W, D] computed transposed (M = D, N = W) so the long side is M
      MM_TRY(launch_gemm_f32({a.u, a.dxd, g->x_proj_w, D, W, (int)T, 1, D, W, 1, 1, D, 0, gp}, st));
      MM_TRY(launch_gemm_f32({a.dxd, wx, a.du, (int)T, D, W, W, 1, D, 1, D, 1, 1}, st));
    }
  }
  {
    StageScope sc(timer, st, MM_STAGE_BWD_CONV);
    MM_TRY(launch_backward_stage(s->io_dtype, a, 5, st));
    MM_TRY(launch_colsum(a.conv_part, (int64_t)B * bw_conv_strips(L), (int64_t)D * 5, cs,
                         a.conv_sum, st));
    MM_TRY(launch_backward_stage(s->io_dtype, a, 7, st));
  }
  return MM_OK;
}

// ---- allocation-free decode step
// Device scratch that stands in for the caller's workspace in
// mamba_mixer_decode_step_noalloc: each GPU the library runs on holds one copy, at its own
// address, until the process ends. The host-side name of the array is not a device address;
// the per-device address comes from hipGetSymbolAddress and is the only one kernels receive.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once per device.
mm_status noalloc_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MM_OK;
}

}  // namespace

extern "C" {

size_t mm_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

mm_status mamba_mixer_decode_step_noalloc(const mm_shape *s, const mm_params *p, const void *xz,
                                          void *y, void *conv_state, float *ssm_state,
                                          void *stream) {
  mm_status r = check_shape(s, true);
  if (r != MM_OK) return r;
  if (layout(*s, true).total > kNoallocScratchBytes) return MM_ERR_WORKSPACE;
  void *ws = nullptr;
  if ((r = noalloc_scratch(&ws)) != MM_OK) return r;
  // every workspace region of the decode step is written before it is read: nothing to clear
  return decode_impl(s, p, xz, y, conv_state, ssm_state, ws, kNoallocScratchBytes, stream,
                     nullptr);
}

size_t mm_layer_workspace_bytes(const mm_shape *s, int32_t d_model) {
  if (!s || check_shape(s, false) != MM_OK || d_model <= 0) return 0;
  return layer_layout(*s, d_model).total;
}

mm_status mamba_layer_prefill(const mm_shape *s, int32_t d_model, const mm_layer_params *p,
                              const void *x, void *out, void *conv_state, float *ssm_state,
                              int states_valid, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return layer_impl(s, d_model, p, x, out, conv_state, ssm_state, states_valid, workspace,
                    workspace_bytes, stream, nullptr);
}

mm_status mamba_layer_prefill_timed(const mm_shape *s, int32_t d_model, const mm_layer_params *p,
                                    const void *x, void *out, void *conv_state, float *ssm_state,
                                    int states_valid, void *workspace, size_t workspace_bytes,
                                    void *stream, mm_stage_timer *timer) {
  return layer_impl(s, d_model, p, x, out, conv_state, ssm_state, states_valid, workspace,
                    workspace_bytes, stream, timer);
}


size_t mm_prefill_workspace_bytes(const mm_shape *s) {
  if (check_shape(s, false) != MM_OK) return 0;
  return layout(*s, false).total;
}

size_t mm_decode_workspace_bytes(const mm_shape *s) {
  if (check_shape(s, true) != MM_OK) return 0;
  return layout(*s, true).total;
}

mm_status mamba_mixer_prefill(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                              void *conv_state, float *ssm_state, int states_valid,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_impl(s, p, xz, y, conv_state, ssm_state, states_valid, workspace,
                      workspace_bytes, stream, nullptr);
}

size_t mm_backward_workspace_bytes(const mm_shape *s) {
  if (check_shape(s, false) != MM_OK || s->dt_rank > 1024 || s->d_state != 16) return 0;
  return bw_layout(*s).total;
}

mm_status mamba_mixer_prefill_backward(const mm_shape *s, const mm_params *p, const void *xz,
                                       const void *dy, const void *conv_state,
                                       const float *ssm_state, int states_valid, const mm_grads *g,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  return backward_impl(s, p, xz, dy, conv_state, ssm_state, states_valid, g, workspace,
                       workspace_bytes, stream, nullptr);
}

mm_status mamba_mixer_prefill_backward_timed(const mm_shape *s, const mm_params *p,
                                             const void *xz, const void *dy,
                                             const void *conv_state, const float *ssm_state,
                                             int states_valid, const mm_grads *g, void *workspace,
                                             size_t workspace_bytes, void *stream,
                                             mm_stage_timer *timer) {
  return backward_impl(s, p, xz, dy, conv_state, ssm_state, states_valid, g, workspace,
                       workspace_bytes, stream, timer);
}

mm_status mamba_mixer_prefill_timed(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                                    void *conv_state, float *ssm_state, int states_valid,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    mm_stage_timer *timer) {
  return prefill_impl(s, p, xz, y, conv_state, ssm_state, states_valid, workspace,
                      workspace_bytes, stream, timer);
}

mm_status mamba_mixer_decode_step(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                                  void *conv_state, float *ssm_state, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  return decode_impl(s, p, xz, y, conv_state, ssm_state, workspace, workspace_bytes, stream,
                     nullptr);
}

mm_status mamba_mixer_decode_step_timed(const mm_shape *s, const mm_params *p, const void *xz,
                                        void *y, void *conv_state, float *ssm_state,
                                        void *workspace, size_t workspace_bytes, void *stream,
                                        mm_stage_timer *timer) {
  return decode_impl(s, p, xz, y, conv_state, ssm_state, workspace, workspace_bytes, stream,
                     timer);
}

mm_stage_timer *mm_stage_timer_create(void) { return new mm_stage_timer(); }

void mm_stage_timer_reset(mm_stage_timer *t) {
  if (!t) return;
  for (auto &r : t->recs) {
    t->pool.push_back(r.a);
    t->pool.push_back(r.b);
  }
  t->recs.clear();
}

void mm_stage_timer_destroy(mm_stage_timer *t) {
  if (!t) return;
  mm_stage_timer_reset(t);
  for (hipEvent_t e : t->pool) (void)hipEventDestroy(e);
  delete t;
}

mm_status mm_stage_timer_read(mm_stage_timer *t, double *ms_sum, int64_t *launches) {
  if (!t || !ms_sum || !launches) return MM_ERR_INVALID_ARG;
  for (int i = 0; i < MM_STAGE_COUNT; ++i) {
    ms_sum[i] = 0.0;
    launches[i] = 0;
  }
  for (auto &r : t->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return MM_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MM_ERR_HIP;
    ms_sum[r.stage] += ms;
    launches[r.stage] += 1;
  }
  return MM_OK;
}

const char *mm_stage_name(int stage) {
  static const char *names[MM_STAGE_COUNT] = {"conv_silu", "x_proj", "rmsnorm", "dt_proj_softplus",
                                              "selective_scan", "conv_state", "layer_rmsnorm",
                                              "in_proj", "out_proj", "bwd_recompute",
                                              "bwd_scan", "bwd_proj", "bwd_conv"};
  return (stage >= 0 && stage < MM_STAGE_COUNT) ? names[stage] : "unknown";
}

const char *mm_status_string(mm_status st) {
  // Callers in C pass any int; in C++ a value outside the enumerators' range may not be read
  // as an mm_status, so the argument's bytes are read as an int.
  int v = 0;
  static_assert(sizeof(v) == sizeof(st), "mm_status is int-sized");
  std::memcpy(&v, &st, sizeof(v));
  switch (v) {
    case MM_OK: return "ok";
    case MM_ERR_INVALID_ARG: return "invalid argument";
    case MM_ERR_UNSUPPORTED: return "unsupported size";
    case MM_ERR_WORKSPACE: return "workspace missing or too small";
    case MM_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int mm_abi_version(void) { return MM_ABI_VERSION; }

}  // extern "C"
