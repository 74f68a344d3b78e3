/*
 * mamba_mixer.h -- C ABI of the MI355X (gfx950) Mamba-1 mixer core.
 *
 * The library computes, on the GPU, the selective-SSM mixer that sits between a Mamba
 * layer's input and output projections:
 *
 *   x, z   = the two halves of the post-in_proj activations xz            (input)
 *   u      = SiLU(causal depthwise conv1d(x) + conv_b)                      (conv + SiLU)
 *   xdbl   = W_x u  = [dt_low | B | C]                                      (x_proj)
 *   dt_low, B, C each RMS-normalised over their own length                  (internal RMSNorm)
 *   dt     = softplus(W_dt dt_low + dt_proj_b)                              (dt_proj)
 *   h_t    = exp(dt A) h_{t-1} + Bbar_t u_t ,  Bbar = dt B (or ZOH)         (selective scan)
 *   y_t    = (C_t . h_t + D u_t) * SiLU(z_t)                                (feed-through + gate)
 *
 * Sources: "Jamba: A Hybrid Transformer-Mamba Language Model" (analysis page of
 * arXiv 2403.19887), section "The Mamba Layer: State-Space Mechanism, Selectivity, and
 * Parallel Scan" -- continuous SSM equation (the D u feed-through), ZOH equation
 * (Abar = exp(Delta A), Bbar), discrete recurrence equation, "From scalar SSM to vector
 * processing" (one scalar SSM per channel), "The selective mechanism" (B, C, Delta from
 * small linear layers of the token), "Parallel training via the parallel scan" (the
 * associative operator that lets the sequence be cut into chunks), "Inference behavior"
 * (O(1) recurrent decode); section "RMSNorm definition and placement" (RMSNorm equation)
 * with "Stabilization: RMSNorm in Mamba layers" (RMSNorm on internal activations).
 * The convolution, SiLU, softplus and gate are the standard Mamba-1 block that page
 * builds on; the pages do not write them out.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller. The
 *     library allocates no device memory in these calls and keeps no state between
 *     calls; scratch space comes from the caller's workspace.
 *   - io_dtype selects the element type of xz, y, conv_state, conv_w, conv_b, x_proj_w
 *     and dt_proj_w (MM_F32: float, MM_BF16: bfloat16 bits in uint16). dt_proj_b, A,
 *     Dskip, the three norm weights and ssm_state are always float.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     return without synchronising the host. States are updated in place in stream order.
 *     y must not alias xz; states must not alias anything else.
 *   - Arguments are validated on the host before anything is launched; on any error
 *     nothing is launched and no output is written. MM_ERR_HIP reports a failed launch;
 *     asynchronous device faults surface at the caller's next synchronisation.
 *   - Entry points are reentrant when given separate workspaces.
 */
#ifndef MAMBA_MIXER_H
#define MAMBA_MIXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MM_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define MM_API __attribute__((visibility("default")))
#else
#define MM_API
#endif

typedef enum {
  MM_OK = 0,
  MM_ERR_INVALID_ARG = -1,   /* NULL required pointer, non-positive size, misalignment */
  MM_ERR_UNSUPPORTED = -2,   /* a size outside this build's limits (see mm_shape)     */
  MM_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than the *_workspace_bytes() */
  MM_ERR_HIP = -4            /* a HIP launch failed                                    */
} mm_status;

typedef enum { MM_F32 = 0, MM_BF16 = 1 } mm_dtype;

/* flags */
enum {
  /* Use the ZOH input matrix of the page's ZOH equation, Bbar = expm1(dt A) / A * B,
     instead of the first-order Bbar = dt * B (the default). */
  MM_FLAG_ZOH_B = 1u << 0,
  /* Scan kernel selection (results agree to fp32 rounding; at most one may be set).
     Default: lanes over (channel, group of d_state / 8 states) when
     batch * d_inner / 64 < 2048 and seqlen > 32, else one lane per (sequence, channel) for
     d_state 16 and a general time-parallel scan (per-range transfers, carries, replay) for
     the other state sizes. Both scan the sequence once, in time order. */
  MM_FLAG_SCAN_SEQUENTIAL = 1u << 1,  /* one lane per (sequence, channel) / the general scan */
  MM_FLAG_SCAN_CHUNKED = 1u << 2,     /* lanes over (channel, state group), 32-token blocks */
  /* Evaluate every exp(dt A[i, n]) directly. Without it the lane kernel checks A on the
     device and, where each lane's states are in arithmetic progression per channel
     (A[i, n0 + k] = A[i, n0] + k delta_i, as for A = -(n + 1)), forms the decays of a lane
     as exp(dt A[i, n0]) times powers of exp(dt delta_i): fewer exps, the same result to fp32
     rounding. First-order Bbar only (ZOH always evaluates each exp). */
  MM_FLAG_SCAN_GENERAL_A = 1u << 3,
  /* Fuse dt_proj + bias + softplus into the scan ("The selective mechanism": Delta from a
     small linear layer of the token): the scan forms dt from the normalised dt_low with the
     same MFMA sequence as the separate dt_proj kernel (the same dt, bit for bit), so the
     [tokens, d_inner] fp32 dt buffer is neither written nor read and the workspace shrinks by
     4 * batch * seqlen * d_inner bytes. It applies to MM_BF16 with d_state 16, dt_rank 256 and
     first-order Bbar where the prefill runs the time-parallel two-pass scan (the default for
     few sequences of more than 32 tokens, or MM_FLAG_SCAN_CHUNKED); elsewhere the flag changes
     nothing. */
  MM_FLAG_FUSED_DTPROJ = 1u << 4
};

/*
 * Problem size. Limits of this build (else MM_ERR_UNSUPPORTED): d_state in {8, 16, 32, 64}
 * (16, the Jamba configuration, runs the tuned projection kernels; every size runs the
 * lane-per-state-group scan where it applies, else the scans named under the flags above;
 * the backward takes 16);
 * 2 <= d_conv <= 4; d_inner % 64 == 0; with MM_BF16, dt_rank % 64 == 0 and
 * d_inner % 128 == 0; with MM_F32, 1 <= dt_rank <= 1024. seqlen >= 1 (prefill),
 * seqlen == 1 (decode). rms_eps > 0 is the RMSNorm epsilon.
 */
typedef struct {
  int32_t batch, seqlen, d_inner, d_state, d_conv, dt_rank;
  mm_dtype io_dtype;
  float rms_eps;
  uint32_t flags;
} mm_shape;

/* Parameters (device pointers, caller-owned, 16-byte aligned). */
typedef struct {
  const void *conv_w;      /* [d_inner, d_conv] io_dtype; tap d_conv-1 multiplies the current token */
  const void *conv_b;      /* [d_inner] io_dtype, or NULL for no bias */
  const void *x_proj_w;    /* [dt_rank + 2*d_state, d_inner] io_dtype; rows = [dt_low | B | C] */
  const void *dt_proj_w;   /* [d_inner, dt_rank] io_dtype */
  const float *dt_proj_b;  /* [d_inner] */
  const float *A;          /* [d_inner, d_state], the (negative real) diagonal state matrix */
  const float *Dskip;      /* [d_inner], the feed-through D */
  const float *dt_norm_w;  /* [dt_rank]  RMSNorm weight of dt_low */
  const float *B_norm_w;   /* [d_state]  RMSNorm weight of B */
  const float *C_norm_w;   /* [d_state]  RMSNorm weight of C */
} mm_params;

/* Bytes of device workspace mamba_mixer_prefill needs for this shape (0 on a bad shape). */
MM_API size_t mm_prefill_workspace_bytes(const mm_shape *s);

/*
 * Chunked long-sequence prefill over `batch` sequences of `seqlen` tokens.
 *   xz          [batch, seqlen, 2*d_inner] io_dtype; x = first d_inner, z = last d_inner
 *   y           [batch, seqlen, d_inner]   io_dtype (before out_proj)
 *   conv_state  [batch, d_inner, d_conv-1] io_dtype, inputs before token 0, oldest first;
 *               on return the last d_conv-1 inputs. NULL: zeros in, nothing out.
 *   ssm_state   [batch, d_inner, d_state] float; on return h after the last token.
 *               NULL: zeros in, nothing out.
 *   states_valid  1: read conv_state / ssm_state as the carried states;
 *                 0: start from zeros (the state buffers, if given, are only written).
 *   workspace   >= mm_prefill_workspace_bytes(s) bytes, 256-byte aligned.
 * Prefill over L1 tokens then over L2 more with the returned states equals one prefill
 * over L1 + L2 tokens (the scan operator is associative).
 */
MM_API mm_status mamba_mixer_prefill(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                              void *conv_state, float *ssm_state, int states_valid,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace mamba_mixer_decode_step needs (s->seqlen must be 1). */
MM_API size_t mm_decode_workspace_bytes(const mm_shape *s);

/*
 * One recurrent token for each of `batch` sequences (the page's O(1) inference step).
 *   xz [batch, 2*d_inner], y [batch, d_inner] io_dtype; conv_state [batch, d_inner, d_conv-1]
 *   and ssm_state [batch, d_inner, d_state] are required and updated in place.
 * N calls equal one prefill over the same N tokens from the same states.
 */
MM_API mm_status mamba_mixer_decode_step(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                                  void *conv_state, float *ssm_state, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * mamba_mixer_decode_step without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the step's intermediates live in a device array inside the library, one per GPU,
 * of mm_noalloc_scratch_bytes() = 64 MiB, held until the process ends. It allocates nothing and
 * calls no allocating routine; results equal mamba_mixer_decode_step's bit for bit (the same
 * kernels). Returns MM_ERR_WORKSPACE when the shape's decode workspace
 * (mm_decode_workspace_bytes) exceeds the array, and the other errors of
 * mamba_mixer_decode_step. Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (other streams, other threads) race and must be serialised by the caller.
 */
MM_API size_t mm_noalloc_scratch_bytes(void);
MM_API mm_status mamba_mixer_decode_step_noalloc(const mm_shape *s, const mm_params *p,
                                                 const void *xz, void *y, void *conv_state,
                                                 float *ssm_state, void *stream);

/*
 * Per-stage timing (a measurement aid). A timer records a pair of HIP events around
 * each kernel stage of every *_timed call on that call's stream; mm_stage_timer_read
 * synchronises on the recorded events and returns the summed milliseconds and the
 * number of timed launches per stage. Stages are listed by mm_stage_name(i),
 * 0 <= i < MM_STAGE_COUNT. A timer is not thread-safe; create one per thread.
 */
enum {
  MM_STAGE_CONV = 0,       /* conv1d + SiLU feeding x_proj */
  MM_STAGE_XPROJ = 1,      /* x_proj contraction */
  MM_STAGE_NORM = 2,       /* RMSNorm of dt_low, B, C */
  MM_STAGE_DTPROJ = 3,     /* dt_proj + bias + softplus */
  MM_STAGE_SCAN = 4,       /* selective scan + D feed-through + SiLU(z) gate + final state */
  MM_STAGE_CONV_STATE = 5, /* conv-state update (only when a conv state is given) */
  MM_STAGE_LAYER_NORM = 6, /* mamba_layer_prefill: RMSNorm of the layer input */
  MM_STAGE_IN_PROJ = 7,    /* mamba_layer_prefill: in_proj */
  MM_STAGE_OUT_PROJ = 8,   /* mamba_layer_prefill: out_proj + residual */
  MM_STAGE_BWD_RECOMPUTE = 9,  /* backward: u, x_proj, the norms, dt_proj's product recomputed */
  MM_STAGE_BWD_SCAN = 10,      /* backward: range transfers, carries, the reverse scan (with the
                                  softplus and gate derivatives), dB / dC */
  MM_STAGE_BWD_PROJ = 11,      /* backward: dt_proj, RMSNorm and x_proj gradients */
  MM_STAGE_BWD_CONV = 12,      /* backward: conv1d + SiLU gradients */
  MM_STAGE_COUNT = 13
};
typedef struct mm_stage_timer mm_stage_timer;
MM_API mm_stage_timer *mm_stage_timer_create(void);
MM_API void mm_stage_timer_destroy(mm_stage_timer *t);
MM_API void mm_stage_timer_reset(mm_stage_timer *t);
MM_API mm_status mm_stage_timer_read(mm_stage_timer *t, double *ms_sum, int64_t *launches);
MM_API const char *mm_stage_name(int stage);

MM_API mm_status mamba_mixer_prefill_timed(const mm_shape *s, const mm_params *p, const void *xz, void *y,
                                    void *conv_state, float *ssm_state, int states_valid,
                                    void *workspace, size_t workspace_bytes, void *stream,
                                    mm_stage_timer *timer);
MM_API mm_status mamba_mixer_decode_step_timed(const mm_shape *s, const mm_params *p, const void *xz,
                                        void *y, void *conv_state, float *ssm_state,
                                        void *workspace, size_t workspace_bytes, void *stream,
                                        mm_stage_timer *timer);

/*
 * Mamba layer around the mixer (bf16 I/O only):
 *     out = x + W_out . mixer(W_in . RMSNorm(x))
 * Jamba analysis page: "RMSNorm definition and placement" (RMSNorm at the input of every Mamba
 * module, RMSNorm equation) and "From scalar SSM to vector processing" (the hidden state is
 * projected to d_inner scalar SSMs whose outputs are projected back). The residual add is the
 * pre-norm block the architecture description implies.
 *   norm_w      [d_model] float, RMSNorm gain of the layer input; norm_eps its epsilon
 *   in_proj_w   [2*d_inner, d_model] bf16; rows 0 .. d_inner-1 give x, the rest z
 *   out_proj_w  [d_model, d_inner] bf16
 *   mixer       the mixer parameters, as for mamba_mixer_prefill
 * Limits (MM_ERR_UNSUPPORTED otherwise): io_dtype MM_BF16, d_model % 128 == 0, and the
 * mixer's own limits.
 */
typedef struct {
  const float *norm_w;
  const void *in_proj_w;
  const void *out_proj_w;
  float norm_eps;
  mm_params mixer;
} mm_layer_params;

/* Bytes of device workspace mamba_layer_prefill needs (0 on a bad shape). */
MM_API size_t mm_layer_workspace_bytes(const mm_shape *s, int32_t d_model);

/*
 * Layer prefill over `batch` sequences of `seqlen` tokens.
 *   x    [batch, seqlen, d_model] bf16 (caller-owned, not modified)
 *   out  [batch, seqlen, d_model] bf16; must not alias x
 *   conv_state, ssm_state, states_valid: as for mamba_mixer_prefill (the mixer's states)
 *   workspace >= mm_layer_workspace_bytes(s, d_model) bytes, 256-byte aligned; it holds the
 *   normalised input, xz and the mixer output besides the mixer's own workspace.
 * Asynchronous on `stream`; on a validation error nothing is launched and nothing written.
 */
MM_API mm_status mamba_layer_prefill(const mm_shape *s, int32_t d_model, const mm_layer_params *p,
                                     const void *x, void *out, void *conv_state, float *ssm_state,
                                     int states_valid, void *workspace, size_t workspace_bytes,
                                     void *stream);
MM_API mm_status mamba_layer_prefill_timed(const mm_shape *s, int32_t d_model,
                                           const mm_layer_params *p, const void *x, void *out,
                                           void *conv_state, float *ssm_state, int states_valid,
                                           void *workspace, size_t workspace_bytes, void *stream,
                                           mm_stage_timer *timer);

/*
 * Backward of the prefill, for training through the parallel scan (Jamba analysis page,
 * "Parallel training via the parallel scan"; the forward is the one of mamba_mixer_prefill,
 * above, with the same shape, flags and parameters). Given the gradient dy of a loss with
 * respect to y, writes the gradients of that loss with respect to xz, every parameter and the
 * two carried states, i.e. the gradients of sum(dy * y):
 *   h_t = Abar_t h_{t-1} + Bbar_t u_t runs backward as dh_t = C_t dys_t + Abar_{t+1} dh_{t+1}
 *   (dys = dy * SiLU(z)); the states h are recomputed from the inputs, never stored by the
 *   forward. Arithmetic is fp32; with bf16 I/O the six products (x_proj, dt_proj and their
 *   input and weight gradients) take each fp32 operand as two bf16 parts, hi + lo (~2^-17
 *   relative), on bf16 MFMA with fp32 accumulation, and dxz is rounded to bf16 on output.
 *   xz, conv_state, ssm_state, states_valid: the forward's inputs (states as they were BEFORE
 *               the forward call; NULL / states_valid 0 = zeros)
 *   dy          [batch, seqlen, d_inner] io_dtype
 *   g           output pointers (all caller-owned device memory, overwritten, not accumulated):
 *               dxz required; the parameter gradients required, except conv_b (required iff
 *               p->conv_b is given); conv_state / ssm_state gradients optional (NULL = skip)
 *   workspace   >= mm_backward_workspace_bytes(s) bytes, 256-byte aligned
 * Limits: those of mamba_mixer_prefill (d_state == 16, 2 <= d_conv <= 4, d_inner % 64 == 0)
 * with 1 <= dt_rank <= 1024 for either io_dtype. The result is deterministic (fixed-order
 * reductions, no atomics).
 */
typedef struct {
  void *dxz;           /* [batch, seqlen, 2*d_inner] io_dtype: d/dx, then d/dz */
  float *conv_w;       /* [d_inner, d_conv] */
  float *conv_b;       /* [d_inner] (NULL when the forward has no conv bias) */
  float *x_proj_w;     /* [dt_rank + 2*d_state, d_inner] */
  float *dt_proj_w;    /* [d_inner, dt_rank] */
  float *dt_proj_b;    /* [d_inner] */
  float *A;            /* [d_inner, d_state] */
  float *Dskip;        /* [d_inner] */
  float *dt_norm_w;    /* [dt_rank] */
  float *B_norm_w;     /* [d_state] */
  float *C_norm_w;     /* [d_state] */
  float *conv_state;   /* [batch, d_inner, d_conv-1] fp32, or NULL */
  float *ssm_state;    /* [batch, d_inner, d_state], or NULL */
} mm_grads;

/* Bytes of device workspace mamba_mixer_prefill_backward needs (0 on a bad shape). */
MM_API size_t mm_backward_workspace_bytes(const mm_shape *s);

MM_API mm_status mamba_mixer_prefill_backward(const mm_shape *s, const mm_params *p,
                                              const void *xz, const void *dy,
                                              const void *conv_state, const float *ssm_state,
                                              int states_valid, const mm_grads *g,
                                              void *workspace, size_t workspace_bytes,
                                              void *stream);
MM_API mm_status mamba_mixer_prefill_backward_timed(const mm_shape *s, const mm_params *p,
                                                    const void *xz, const void *dy,
                                                    const void *conv_state,
                                                    const float *ssm_state, int states_valid,
                                                    const mm_grads *g, void *workspace,
                                                    size_t workspace_bytes, void *stream,
                                                    mm_stage_timer *timer);

MM_API const char *mm_status_string(mm_status st);
MM_API int mm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MAMBA_MIXER_H */
