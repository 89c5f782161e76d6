/* Plain C client of the verification library: compiled with gcc against
 * include/spec_verify.h and linked to libspecverify.so by
 * tests/test_c_client.py. Exercises only host-side behaviour (sizes,
 * argument errors, error text), so it runs without a GPU: every call below
 * fails its host checks before any device work. Exit status 0 on success. */
#include <stdio.h>
#include <string.h>

#include "spec_verify.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  /* workspace sizes: positive, 256-byte multiples, 0 for invalid sizes */
  size_t ws = spec_verify_workspace_bytes(64, 512, 128256, 0, 1.0f);
  if (ws == 0 || ws % 256 != 0) {
    fprintf(stderr, "bad workspace size %zu\n", ws);
    ++failures;
  }
  expect(spec_verify_workspace_bytes(-1, 0, 10, 0, 1.0f) == 0, 1, "negative B gives 0");
  expect(spec_verify_workspace_bytes(64, 512, 128256, 50, 0.9f) > ws, 1, "top-k adds records");

  /* error text for every code, and for an unknown one */
  const int codes[] = {SV_OK, SV_EINVAL, SV_EDTYPE, SV_EWORKSPACE, SV_EHIP, SV_EUNSUPPORTED,
                       SV_SEQ_BAD_TOKEN, SV_SEQ_BAD_ROW, SV_SEQ_BAD_OFFSETS, SV_SEQ_SYNC_TIMEOUT};
  for (size_t i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
    const char* t = spec_verify_strerror(codes[i]);
    if (t == NULL || t[0] == '\0') {
      fprintf(stderr, "no text for code %d\n", codes[i]);
      ++failures;
    }
  }
  expect(strcmp(spec_verify_strerror(12345), "unknown code"), 0, "unknown code text");
  expect(spec_verify_num_stages(0, 1.0f), 1, "one kernel without filters");
  expect(spec_verify_num_stages(50, 0.9f), 3, "three kernels with filters");

  /* host-side argument errors (fake device pointers are never dereferenced) */
  void* p = (void*)0x1000;
  void* w = (void*)0x10000;
  int32_t* ip = (int32_t*)p;
  float* fp = (float*)p;
  expect(spec_verify(p, p, ip, fp, 4, 4, 1024, 1.0f, 0, 1.0f, (sv_dtype)7, ip, ip, w, 16, NULL),
         SV_EDTYPE, "bad dtype");
  expect(spec_verify(p, p, ip, fp, 4, 65, 1024, 1.0f, 0, 1.0f, SV_BF16, ip, ip, w, 16, NULL),
         SV_EINVAL, "K above 64");
  expect(spec_verify(p, p, ip, fp, 4, 4, 1024, -1.0f, 0, 1.0f, SV_BF16, ip, ip, w, 16, NULL),
         SV_EINVAL, "negative temperature");
  expect(spec_verify(p, p, ip, fp, 4, 4, 1024, 1.0f, 0, 1.5f, SV_BF16, ip, ip, w, 16, NULL),
         SV_EINVAL, "top_p above 1");
  expect(spec_verify(p, p, ip, fp, 4, 4, 1024, 1.0f, 0, 1.0f, SV_BF16, ip, ip, w, 16, NULL),
         SV_EWORKSPACE, "workspace too small");
  expect(spec_verify(p, p, ip, fp, 4, 4, 4096, 1.0f, 2000, 1.0f, SV_BF16, ip, ip, w, 16, NULL),
         SV_EUNSUPPORTED, "top_k above the limit");
  expect(spec_verify(NULL, NULL, NULL, NULL, 0, 4, 1024, 1.0f, 0, 1.0f, SV_BF16, NULL, NULL, NULL,
                     0, NULL),
         SV_OK, "empty batch");
  expect(spec_verify_ragged(p, p, ip, fp, NULL, NULL, 4, 10, 1000, 1.0f, 0, 1.0f, SV_BF16, ip, ip,
                            w, 16, NULL),
         SV_EINVAL, "ragged without offsets");
  expect(spec_verify_accept_stats(p, p, NULL, 4, 12, 1000, 0.0f, 0, 1.0f, SV_BF16, fp, fp, w, 16,
                                  NULL),
         SV_EINVAL, "acceptance statistics at temperature 0");
  expect(spec_verify_accept_stats(p, p, NULL, 4, 13, 1000, 1.0f, 0, 1.0f, SV_BF16, fp, fp, w, 16,
                                  NULL),
         SV_EINVAL, "draft rows not a multiple of B");
  expect(spec_verify_accept_stats(p, p, NULL, 4, 12, 1000, 1.0f, 0, 0.9f, SV_BF16, fp, fp, w, 16,
                                  NULL),
         SV_EWORKSPACE, "top-p alone reaches the workspace check");
  if (failures == 0) printf("c client ok\n");
  return failures == 0 ? 0 : 1;
}
