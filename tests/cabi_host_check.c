// Host-side exercise of the C ABI for the sanitizer build: workspace sizing
// for valid and invalid arguments, rejection of null pointers and small
// workspaces, the timing hook and the error string.  Every call here fails
// validation or only sizes, so no kernel is launched and no GPU is needed.
// Exit status 0 when every return code is the documented one.
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/sparsepr.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "line %d: %s failed\n", __LINE__, #cond);   \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

int main() {
  static char fake_buf[64];
  void* F = fake_buf;   // never dereferenced: every call below fails validation first
  EXPECT(strncmp(sparsepr_version(), "sparsepr-gfx950", 15) == 0);

  const int d_values[] = {64, 128, 96};
  for (int di = 0; di < 3; ++di) {
    sparsepr_shape s = {4, 8192, d_values[di], SPARSEPR_BF16, 0.0f};
    sparsepr_partition_params pp = {32, 32, 256, 16, 8, 8, 0.5, 0, 0};
    sparsepr_route_params rp = {0, 0.25, 128};
    sparsepr_fit_params fp = {128, 16, 1e-3};
    const size_t n = sparsepr_workspace_size(&s, &pp, &rp, &fp);
    if (d_values[di] == 96) {
      EXPECT(n == 0 && strlen(sparsepr_last_error()) > 0);
      continue;
    }
    EXPECT(n > 0 && strlen(sparsepr_last_error()) == 0);
    // each field pushed out of range in turn
    sparsepr_partition_params bad = pp;
    bad.G_k = 0; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    bad = pp; bad.G_q = 9000; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    bad = pp; bad.M_s = 0; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    bad = pp; bad.r_k = s.d + 1; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    bad = pp; bad.iters_q = 0; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    bad = pp; bad.semantic = 2; EXPECT(sparsepr_workspace_size(&s, &bad, &rp, &fp) == 0);
    sparsepr_route_params rb = rp;
    rb.density = 0.0; EXPECT(sparsepr_workspace_size(&s, &pp, &rb, &fp) == 0);
    rb = rp; rb.M = -1; EXPECT(sparsepr_workspace_size(&s, &pp, &rb, &fp) == 0);
    sparsepr_fit_params fb = fp;
    fb.rank = s.d + 1; EXPECT(sparsepr_workspace_size(&s, &pp, &rp, &fb) == 0);
    fb = fp; fb.lambda = -1.0; EXPECT(sparsepr_workspace_size(&s, &pp, &rp, &fb) == 0);
    fb = fp; fb.lambda = 0.0; fb.M = s.d; EXPECT(sparsepr_workspace_size(&s, &pp, &rp, &fb) == 0);
    fb = fp; fb.lambda = 0.0; fb.M = s.d + 1; EXPECT(sparsepr_workspace_size(&s, &pp, &rp, &fb) > 0);
    sparsepr_shape sb = s;
    sb.N = 0; EXPECT(sparsepr_workspace_size(&sb, &pp, &rp, &fp) == 0);
    sb = s; sb.scale = -1.0f; EXPECT(sparsepr_workspace_size(&sb, &pp, &rp, &fp) == 0);
    EXPECT(sparsepr_workspace_size(NULL, &pp, &rp, &fp) == 0);
    EXPECT(sparsepr_workspace_size(&s, NULL, &rp, &fp) == 0);

    // entry points: null pointers, then a workspace one byte short
    EXPECT(sparsepr_partition(&s, &pp, NULL, F, F, F, F, F, F, F, F, F, F, F, F, F, F, F, n, NULL) ==
           SPARSEPR_EINVAL);
    EXPECT(sparsepr_partition(&s, &pp, F, F, F, F, F, F, F, F, F, F, F, F, F, F, F, F, 16, NULL) ==
           SPARSEPR_EWORKSPACE);
    EXPECT(sparsepr_route(&s, &pp, &rp, NULL, F, (const double*)F, (const double*)F, (int32_t*)F, (int32_t*)F,
                          (int64_t*)F, F, n, NULL) == SPARSEPR_EINVAL);
    EXPECT(sparsepr_route(&s, &pp, &rp, (const int32_t*)F, (const int32_t*)F, (const double*)F, (const double*)F,
                          (int32_t*)F, (int32_t*)F, (int64_t*)F, F, 8, NULL) == SPARSEPR_EWORKSPACE);
    EXPECT(sparsepr_route_noalloc(&s, &pp, &rp, NULL, (const int32_t*)F, (const double*)F, (const double*)F,
                                  (int32_t*)F, (int32_t*)F, (int64_t*)F, NULL) == SPARSEPR_EINVAL);
    EXPECT(sparsepr_attend(&s, &pp, F, F, F, (const int32_t*)F, (const int32_t*)F, (const int32_t*)F,
                           (const int32_t*)F, NULL, (float*)F, F, n, NULL) == SPARSEPR_EINVAL);
    EXPECT(sparsepr_probe_fit(&s, &pp, &fp, F, F, F, (const int32_t*)F, (const int32_t*)F, (const int32_t*)F,
                              (const double*)F, NULL, (int32_t*)F, (double*)F, (float*)F, (double*)F, (double*)F,
                              (double*)F, (double*)F, (int32_t*)F, F, n, NULL) == SPARSEPR_EINVAL);
    EXPECT(sparsepr_correct(&s, &fp, (const float*)F, (const int32_t*)F, (const int32_t*)F, (const float*)F,
                            (const double*)F, (const double*)F, (const double*)F, (const double*)F, (const int32_t*)F,
                            NULL, F, n, NULL) == SPARSEPR_EINVAL);
    const size_t dn = sparsepr_dense_workspace_size(&s);
    EXPECT(dn >= (size_t)2 * s.H * s.N * s.d);
    EXPECT(sparsepr_dense_attend(&s, F, F, F, F, (float*)F, F, dn - 1, NULL) == SPARSEPR_EWORKSPACE);
    EXPECT(sparsepr_dense_attend(&s, F, F, NULL, F, (float*)F, F, dn, NULL) == SPARSEPR_EINVAL);
  }

  // a fit with no probes does nothing and succeeds without any pointer
  {
    sparsepr_shape s = {2, 1024, 64, SPARSEPR_F32, 0.0f};
    sparsepr_partition_params pp = {8, 8, 64, 16, 8, 8, 0.5, 0, 0};
    sparsepr_fit_params fp = {0, 8, 1e-3};
    EXPECT(sparsepr_probe_fit(&s, &pp, &fp, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                              NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                              NULL) == SPARSEPR_OK);
  }
  // the static scratch of the allocation-free route holds 2^22 cells
  {
    sparsepr_shape s = {5, 8192, 64, SPARSEPR_BF16, 0.0f};
    sparsepr_partition_params pp = {1024, 1024, 256, 16, 8, 8, 0.5, 0, 0};
    sparsepr_route_params rp = {0, 0.25, 128};
    EXPECT(sparsepr_route_noalloc(&s, &pp, &rp, (const int32_t*)F, (const int32_t*)F, (const double*)F,
                                  (const double*)F, (int32_t*)F, (int32_t*)F, (int64_t*)F, NULL) ==
           SPARSEPR_EWORKSPACE);
    EXPECT(strstr(sparsepr_last_error(), "static scratch") != NULL);
  }
  // the eigensolver's sizing and validation
  EXPECT(sparsepr_sym_eigen_workspace_size(0, 64) == 0);
  EXPECT(sparsepr_sym_eigen_workspace_size(3, 96) == 0);
  {
    const size_t n = sparsepr_sym_eigen_workspace_size(3, 128);
    EXPECT(n >= (size_t)3 * 128 * 128 * 8);
    EXPECT(sparsepr_sym_eigen(3, 128, 0, (const double*)F, (double*)F, (double*)F, F, n, NULL) ==
           SPARSEPR_EINVAL);
    EXPECT(sparsepr_sym_eigen(3, 128, 4, (const double*)F, (double*)F, (double*)F, F, n - 1, NULL) ==
           SPARSEPR_EWORKSPACE);
  }
  // the timing hook never touches the device
  EXPECT(sparsepr_attend_kernel_timing(1) == SPARSEPR_OK);
  double ms = -1.0;
  int launches = -1;
  EXPECT(sparsepr_attend_kernel_time(&ms, &launches) == SPARSEPR_OK && ms == 0.0 && launches == 0);
  EXPECT(sparsepr_attend_kernel_time(NULL, &launches) == SPARSEPR_EINVAL);
  EXPECT(sparsepr_attend_kernel_timing(0) == SPARSEPR_OK);
  EXPECT(sparsepr_mfma_rate_probe(0, 10, (float*)F, NULL) == SPARSEPR_EINVAL);
  EXPECT(sparsepr_tile_rate_probe(0, 10, (float*)F, NULL) == SPARSEPR_EINVAL);
  EXPECT(sparsepr_tile_rate_probe(4, 10, NULL, NULL) == SPARSEPR_EINVAL);

  if (g_fail) fprintf(stderr, "%d checks failed\n", g_fail);
  else printf("all host checks passed\n");
  return g_fail ? 1 : 0;
}
