/* A plain C99 client of the C ABI (no GPU needed): includes the public
 * headers, links libaxr.so, solves a codebook and checks that invalid
 * arguments are rejected with a message before any device call.  Prints
 * one line per check and exits nonzero on the first failure. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "axr.h"
#include "axr_probe.h"

static int fails = 0;

static void check(int cond, const char* what) {
  printf("%s %s\n", cond ? "ok" : "FAIL", what);
  if (!cond) ++fails;
}

int main(void) {
  double c[16], t[15];
  check(axr_version() >= 10000, "version");
  check(axr_codebook(128, 3, c, t) == AXR_OK, "codebook d=128 b=3");
  /* symmetric, ascending, middle threshold exactly 0, thresholds at midpoints */
  int sym = 1, asc = 1, mid = 1;
  for (int i = 0; i < 8; ++i) sym &= c[i] == -c[7 - i];
  for (int i = 0; i + 1 < 8; ++i) asc &= c[i] < c[i + 1];
  for (int i = 0; i < 7; ++i) mid &= fabs(t[i] - 0.5 * (c[i] + c[i + 1])) < 1e-15;
  check(sym && asc && mid && t[3] == 0.0, "codebook structure");
  /* b = 1: centroids +-sigma sqrt(2/pi) */
  check(axr_codebook(64, 1, c, t) == AXR_OK &&
            fabs(c[1] - sqrt(2.0 / acos(-1.0)) / 8.0) < 1e-14 && t[0] == 0.0,
        "codebook b=1 closed form");
  check(axr_codebook(0, 3, c, t) == AXR_EINVAL && strstr(axr_last_error(), "d=0") != NULL,
        "codebook rejects d=0");
  uint32_t signs[4] = {0, 0, 0, 0};
  check(axr_quantize_keys((const void*)0, AXR_F16, 10, 100, 3, signs, (uint32_t*)0, (float*)0,
                          (void*)0) == AXR_EUNSUPPORTED,
        "quantize rejects d=100");
  check(axr_quantize_keys((const void*)0, AXR_F16, 0, 128, 3, signs, (uint32_t*)0, (float*)0,
                          (void*)0) == AXR_OK,
        "quantize n=0 is a no-op");
  check(axr_score((const void*)0, AXR_F32, (const uint32_t*)0, (const float*)0, signs, 1, 3, 2,
                  16, 16, 128, 3, (float*)0, (void*)0) == AXR_EINVAL &&
            strstr(axr_last_error(), "multiple") != NULL,
        "score rejects Hq % Hkv != 0");
  check(axr_probe_read_stream((const void*)0, 16, (uint32_t*)0, (void*)0) != 0,
        "probe rejects null buffers");
  return fails ? 1 : 0;
}
