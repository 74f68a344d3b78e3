// Host-only driver (C11, as a C caller of the ABI) of the validation layer, built with
// AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py). Every call below either sizes a
// workspace or fails validation before anything is launched, so it runs without a GPU; the
// sanitizers check the host code on those paths (shape checks, workspace layouts, status and
// stage tables, the stage timer, the allocation-free entry point's size check).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mamba_mixer.h"

static int g_fail = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static mm_shape shape(int b, int l, int d, int n, int k, int r, int dt, uint32_t flags) {
  mm_shape s;
  s.batch = b;
  s.seqlen = l;
  s.d_inner = d;
  s.d_state = n;
  s.d_conv = k;
  s.dt_rank = r;
  s.io_dtype = (mm_dtype)dt;   // C: any int (7 below is out of range on purpose)
  s.rms_eps = 1e-6f;
  s.flags = flags;
  return s;
}

int main() {
  EXPECT(mm_abi_version() > 0);
  for (int v = -6; v <= 1; ++v) EXPECT(mm_status_string((mm_status)v) != NULL);
  for (int i = -2; i < MM_STAGE_COUNT + 2; ++i) (void)mm_stage_name(i);
  EXPECT(mm_stage_name(MM_STAGE_SCAN) != NULL);

  // workspace sizes: valid shapes size > 0, invalid ones 0
  const mm_shape ok = shape(1, 4096, 8192, 16, 4, 256, MM_BF16, 0);
  EXPECT(mm_prefill_workspace_bytes(&ok) > 0);
  EXPECT(mm_prefill_workspace_bytes(NULL) == 0);
  const int sizes[4] = {8, 16, 32, 64};
  for (int i = 0; i < 4; ++i) {
    const int n = sizes[i];
    const mm_shape s = shape(2, 1100, 256, n, 4, 64, MM_BF16, 0);
    EXPECT(mm_prefill_workspace_bytes(&s) > 0);
    const mm_shape s2 = shape(2, 1100, 256, n, 4, 64, MM_BF16, MM_FLAG_SCAN_SEQUENTIAL);
    EXPECT(mm_prefill_workspace_bytes(&s2) > 0);
  }
  const mm_shape big = shape(1, 131072, 8192, 16, 4, 256, MM_BF16, 0);
  EXPECT(mm_prefill_workspace_bytes(&big) > mm_prefill_workspace_bytes(&ok));
  const mm_shape dec = shape(256, 1, 8192, 16, 4, 256, MM_BF16, 0);
  EXPECT(mm_decode_workspace_bytes(&dec) > 0);
  EXPECT(mm_decode_workspace_bytes(&ok) == 0);          // decode needs seqlen 1
  EXPECT(mm_layer_workspace_bytes(&ok, 4096) > 0);
  EXPECT(mm_layer_workspace_bytes(&ok, 0) == 0);
  EXPECT(mm_backward_workspace_bytes(&ok) > 0);
  const mm_shape bad[] = {
      shape(0, 16, 256, 16, 4, 64, MM_BF16, 0),    shape(1, -3, 256, 16, 4, 64, MM_BF16, 0),
      shape(1, 16, 96, 16, 4, 64, MM_BF16, 0),     shape(1, 16, 256, 12, 4, 64, MM_BF16, 0),
      shape(1, 16, 256, 16, 5, 64, MM_BF16, 0),    shape(1, 16, 256, 16, 4, 100, MM_BF16, 0),
      shape(1, 16, 256, 16, 4, 64, 7, 0), shape(1, 16, 256, 16, 4, 64, MM_BF16, 1u << 9),
      shape(1, 16, 256, 16, 4, 64, MM_BF16, MM_FLAG_SCAN_SEQUENTIAL | MM_FLAG_SCAN_CHUNKED),
      shape(1 << 20, 1 << 20, 8192, 16, 4, 256, MM_BF16, 0)};
  for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    EXPECT(mm_prefill_workspace_bytes(&bad[i]) == 0);
    EXPECT(mm_backward_workspace_bytes(&bad[i]) == 0);
  }

  // entry points reject bad arguments before any launch
  void *f = (void *)(uintptr_t)0x100000;
  mm_params p;
  p.conv_w = p.conv_b = p.x_proj_w = p.dt_proj_w = f;
  p.dt_proj_b = p.A = p.Dskip = p.dt_norm_w = p.B_norm_w = p.C_norm_w = (const float *)f;
  const size_t need = mm_prefill_workspace_bytes(&ok);
  void *f2 = (void *)(uintptr_t)0x200000;
  EXPECT(mamba_mixer_prefill(NULL, &p, f, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, NULL, f, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, &p, NULL, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, &p, f, f, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, &p, (char *)f + 2, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, &p, f, f2, NULL, NULL, 2, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_prefill(&ok, &p, f, f2, NULL, NULL, 0, f, need - 1, NULL) ==
         MM_ERR_WORKSPACE);
  EXPECT(mamba_mixer_prefill(&ok, &p, f, f2, NULL, NULL, 0, NULL, need, NULL) ==
         MM_ERR_WORKSPACE);
  EXPECT(mamba_mixer_prefill(&bad[3], &p, f, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_UNSUPPORTED);
  mm_params p2 = p;
  p2.A = NULL;
  EXPECT(mamba_mixer_prefill(&ok, &p2, f, f2, NULL, NULL, 0, f, need, NULL) ==
         MM_ERR_INVALID_ARG);
  const size_t needd = mm_decode_workspace_bytes(&dec);
  EXPECT(mamba_mixer_decode_step(&dec, &p, f, f2, NULL, (float *)f, f, needd, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_mixer_decode_step(&dec, &p, f, f2, f, (float *)f, f, needd - 1, NULL) ==
         MM_ERR_WORKSPACE);
  // the allocation-free decode step: a shape beyond its scratch is refused before any HIP call
  const mm_shape huge = shape(4096, 1, 16384, 16, 4, 512, MM_BF16, 0);
  EXPECT(mm_decode_workspace_bytes(&huge) > mm_noalloc_scratch_bytes());
  EXPECT(mamba_mixer_decode_step_noalloc(&huge, &p, f, f2, f, (float *)f, NULL) ==
         MM_ERR_WORKSPACE);
  EXPECT(mamba_mixer_decode_step_noalloc(&ok, &p, f, f2, f, (float *)f, NULL) ==
         MM_ERR_INVALID_ARG);
  mm_layer_params lp;
  lp.mixer = p;
  lp.norm_w = (const float *)f;
  lp.in_proj_w = lp.out_proj_w = f;
  lp.norm_eps = 1e-6f;
  const size_t needl = mm_layer_workspace_bytes(&ok, 4096);
  EXPECT(mamba_layer_prefill(&ok, 4096, &lp, f, f, NULL, NULL, 0, f, needl, NULL) ==
         MM_ERR_INVALID_ARG);
  EXPECT(mamba_layer_prefill(&ok, 100, &lp, f, f2, NULL, NULL, 0, f, needl, NULL) ==
         MM_ERR_UNSUPPORTED);
  EXPECT(mamba_mixer_prefill_backward(&ok, &p, f, f2, NULL, NULL, 0, NULL, f,
                                      mm_backward_workspace_bytes(&ok), NULL) ==
         MM_ERR_INVALID_ARG);

  // the stage timer with nothing recorded
  mm_stage_timer *t = mm_stage_timer_create();
  EXPECT(t != NULL);
  double ms[MM_STAGE_COUNT];
  int64_t n[MM_STAGE_COUNT];
  mm_stage_timer_reset(t);
  EXPECT(mm_stage_timer_read(t, ms, n) == MM_OK);
  for (int i = 0; i < MM_STAGE_COUNT; ++i) EXPECT(n[i] == 0);
  mm_stage_timer_destroy(t);

  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("host validation checks passed\n");
  return 0;
}
