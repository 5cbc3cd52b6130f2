/*
 * Drives the host layer of libkda (argument checks, workspace sizing, status
 * strings, timing bookkeeping) through every path that returns before a HIP call,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer on the host side.
 * No GPU is needed: device pointers are fake, aligned addresses the host never
 * dereferences. Exit status 0 when every call returned what the header promises.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kda.h"

static int failures = 0;

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      printf("FAIL line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, want); \
      ++failures;                                                                       \
    } else if ((want) != KDA_OK && kda_last_error()[0] == '\0') {                       \
      printf("FAIL line %d: %s left no error message\n", __LINE__, #call);             \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

#define F ((void *)(uintptr_t)(1u << 20))
#define FF ((float *)(uintptr_t)(1u << 20))
#define MIS ((void *)(uintptr_t)((1u << 20) + 4))

static int fwd(const void *q, const float *la, const float *s0, const int32_t *cu, int num_seqs, void *o, int B,
               int T, int H, int dk, int chunk, int dtype, void *ws, size_t ws_bytes) {
  return kda_chunk_fwd(q, F, F, la, FF, s0, cu, num_seqs, o, FF, B, T, H, dk, 128, chunk, dtype, ws, ws_bytes, NULL);
}

int main(void) {
  if (kda_abi_version() != KDA_ABI_VERSION) {
    printf("FAIL: ABI version %d != %d\n", kda_abi_version(), KDA_ABI_VERSION);
    ++failures;
  }
  for (int s = -8; s <= 3; ++s)
    if (strlen(kda_status_string(s)) == 0) ++failures;

  /* prefill: every rejection */
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 64, 2, 64, 64, KDA_BF16, NULL, 0), KDA_ERR_UNSUPPORTED);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 64, 2, 128, 32, KDA_BF16, NULL, 0), KDA_ERR_UNSUPPORTED);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 64, 2, 128, 64, 7, NULL, 0), KDA_ERR_UNSUPPORTED);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, -1, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 64, 0, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(NULL, FF, NULL, NULL, 0, F, 1, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, NULL, NULL, NULL, 0, F, 1, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(MIS, FF, NULL, NULL, 0, F, 1, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, (const float *)MIS, NULL, 0, F, 1, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, NULL, (const int32_t *)F, 2, F, 2, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, NULL, (const int32_t *)F, 0, F, 1, 10, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 64, 2, 128, 64, KDA_BF16, F, 16), KDA_ERR_WORKSPACE);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1 << 16, 1 << 16, 2, 128, 64, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(F, FF, NULL, NULL, 0, F, 1, 1 << 30, 64, 128, 16, KDA_BF16, NULL, 0), KDA_ERR_INVALID_ARG);
  EXPECT(fwd(NULL, NULL, NULL, NULL, 0, NULL, 0, 64, 2, 128, 64, KDA_BF16, NULL, 0), KDA_OK);

  /* workspace queries over a grid of shapes, every path; fused checks */
  const int Bs[] = {0, 1, 3}, Ts[] = {0, 1, 15, 16, 63, 64, 65, 4096, 131072}, Hs[] = {1, 2, 32, 64};
  size_t total = 0;
  for (int a = 0; a < 3; ++a)
    for (int b = 0; b < 9; ++b)
      for (int c = 0; c < 4; ++c)
        for (int chunk = 16; chunk <= 64; chunk += 48)
          for (int dtype = 0; dtype <= 1; ++dtype) {
            total += kda_chunk_fwd_workspace_size(Bs[a], Ts[b], Hs[c], 0, chunk, dtype);
            total += kda_chunk_fwd_workspace_size(1, Ts[b], Hs[c], 3, chunk, dtype);
            for (int path = KDA_PATH_AUTO; path <= KDA_PATH_RECORD_SEGMENTED; ++path) {
              kda_fusion f;
              memset(&f, 0, sizeof f);
              f.prefill_path = path;
              total += kda_chunk_fwd_fused_workspace_size(Bs[a], Ts[b], Hs[c], 0, chunk, dtype, &f);
            }
            total += kda_chunk_bwd_workspace_size(Bs[a], Ts[b], Hs[c], 0, dtype);
            total += kda_dplr_chunk_fwd_workspace_size(Bs[a], Ts[b], Hs[c], 0, dtype);
          }
  if (total == 0) ++failures;
  kda_fusion bad;
  memset(&bad, 0, sizeof bad);
  bad.prefill_path = 9;
  EXPECT(kda_chunk_fwd_fused(F, F, F, FF, FF, NULL, NULL, 0, F, FF, 1, 64, 2, 128, 128, 64, KDA_BF16, &bad, NULL, 0,
                             NULL), KDA_ERR_INVALID_ARG);
  memset(&bad, 0, sizeof bad);
  bad.qk_eps = -1.f;
  EXPECT(kda_chunk_fwd_fused(F, F, F, FF, FF, NULL, NULL, 0, F, FF, 1, 64, 2, 128, 128, 64, KDA_BF16, &bad, NULL, 0,
                             NULL), KDA_ERR_INVALID_ARG);
  memset(&bad, 0, sizeof bad);
  bad.out_gate = F;
  EXPECT(kda_chunk_fwd_fused(F, F, F, FF, FF, NULL, NULL, 0, F, FF, 1, 64, 2, 128, 128, 64, KDA_BF16, &bad, NULL, 0,
                             NULL), KDA_ERR_INVALID_ARG);
  if (kda_chunk_fwd_fused_workspace_size(1, 64, 2, 0, 64, KDA_BF16, &bad) != 0) ++failures;

  /* the no-alloc prefill: every check, the scratch limit included, before any HIP call */
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, FF, FF, NULL, NULL, 0, F, FF, 12, 64, 32, 128, 128, 64, KDA_BF16, NULL),
         KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, FF, FF, NULL, NULL, 0, F, FF, 1, 65536, 32, 128, 128, 16, KDA_FP32, NULL),
         KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, FF, FF, NULL, NULL, 0, MIS, FF, 1, 64, 2, 128, 128, 64, KDA_BF16, NULL),
         KDA_ERR_INVALID_ARG);

  /* decode, epilogue, backward and DPLR rejections */
  EXPECT(kda_decode_step(F, F, F, FF, FF, FF, F, 4, 2, 96, 128, KDA_BF16, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_decode_step(F, F, F, FF, FF, NULL, F, 4, 2, 128, 128, KDA_BF16, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_decode_step(F, F, F, FF, FF, FF, F, -1, 2, 128, 128, KDA_BF16, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_decode_step(F, F, F, FF, FF, FF, F, 0, 2, 128, 128, KDA_BF16, NULL), KDA_OK);
  EXPECT(kda_output_norm_gate(F, F, FF, F, 4, 64, 1e-6f, KDA_BF16, NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_output_norm_gate(NULL, F, FF, F, 4, 128, 1e-6f, KDA_BF16, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_output_norm_gate(F, F, FF, F, 0, 128, 1e-6f, KDA_BF16, NULL), KDA_OK);
  EXPECT(kda_chunk_bwd(F, F, F, FF, FF, NULL, NULL, 0, F, NULL, F, F, F, FF, FF, FF, 1, 64, 2, 128, 128, 3, NULL, 0,
                       NULL), KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_bwd(F, F, F, FF, FF, NULL, NULL, 0, NULL, NULL, F, F, F, FF, FF, FF, 1, 64, 2, 128, 128, KDA_BF16,
                       NULL, 0, NULL), KDA_ERR_INVALID_ARG);
  EXPECT(kda_chunk_bwd(F, F, F, FF, FF, NULL, NULL, 0, F, NULL, F, F, F, FF, FF, FF, 1, 64, 2, 128, 128, KDA_BF16, F,
                       16, NULL), KDA_ERR_WORKSPACE);
  EXPECT(kda_dplr_chunk_fwd(F, F, F, F, F, FF, NULL, NULL, 0, F, FF, 1, 64, 2, 128, 128, 16, KDA_BF16, NULL, 0, NULL),
         KDA_ERR_UNSUPPORTED);
  EXPECT(kda_dplr_chunk_fwd(F, F, F, NULL, F, FF, NULL, NULL, 0, F, FF, 1, 64, 2, 128, 128, 64, KDA_BF16, NULL, 0,
                            NULL), KDA_ERR_INVALID_ARG);

  /* timing bookkeeping without any recorded event */
  double ms[16];
  int cnt[16];
  EXPECT(kda_timing_enable(1), KDA_OK);
  EXPECT(kda_timing_read(ms, cnt, 16), KDA_OK);
  EXPECT(kda_timing_read(ms, cnt, -1), KDA_ERR_INVALID_ARG);
  EXPECT(kda_timing_enable(0), KDA_OK);

  printf("%d failures\n", failures);
  return failures != 0;
}
