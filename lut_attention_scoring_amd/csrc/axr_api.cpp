// C-ABI layer: argument validation, error reporting, codebook preparation and
// kernel dispatch.  Every check runs before the first HIP call, so rejected
// calls never touch the device.  See include/axr.h for the contract.

#include "axr.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <string>

#include "axr_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return AXR_OK;
}

bool supported_d(int d) { return d == 128 || d == 256 || d == 512; }
bool supported_b(int b) { return b >= 2 && b <= 4; }
bool supported_dtype(int t) { return t == AXR_F32 || t == AXR_F16 || t == AXR_BF16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int d, int b, int dtype, const uint32_t* sign_bits) {
  if (!supported_d(d)) return fail(AXR_EUNSUPPORTED, "d=%d is not supported (128, 256, 512)", d);
  if (!supported_b(b)) return fail(AXR_EUNSUPPORTED, "b=%d is not supported (2, 3, 4)", b);
  if (!supported_dtype(dtype)) return fail(AXR_EUNSUPPORTED, "dtype=%d is not supported", dtype);
  if (sign_bits == nullptr) return fail(AXR_EINVAL, "sign_bits is null");
  return AXR_OK;
}

void fill_signs(uint32_t* dst, const uint32_t* sign_bits, int d) {
  std::memset(dst, 0, sizeof(uint32_t) * axr::kMaxSignWords);
  std::memcpy(dst, sign_bits, sizeof(uint32_t) * (d / 32));
}

int hip_status(int err, const char* what) {
  if (err != 0) return fail(AXR_EHIP, "%s: HIP error %d", what, err);
  return ok();
}

}  // namespace

extern "C" {

int axr_version(void) { return 10000; }

const char* axr_last_error(void) { return g_last_error.c_str(); }

int axr_codebook(int d, int b, double* centroids, double* thresholds) {
  if (d < 1) return fail(AXR_EINVAL, "d=%d must be >= 1", d);
  if (b < 1 || b > 4) return fail(AXR_EINVAL, "b=%d must be in [1, 4]", b);
  if (centroids == nullptr || thresholds == nullptr)
    return fail(AXR_EINVAL, "centroids and thresholds must be non-null");
  const axr::Codebook& cb = axr::cached_codebook(d, b);
  const int levels = 1 << b;
  for (int i = 0; i < levels; ++i) centroids[i] = cb.centroid[i];
  for (int i = 0; i + 1 < levels; ++i) thresholds[i] = cb.threshold[i];
  return ok();
}

static int write_common(const void* x, int dtype, int64_t n, int d, int b,
                        const uint32_t* sign_bits, uint32_t* packed, float* norms, float* y,
                        int mode, void* stream, const int32_t* pos = nullptr,
                        int64_t t_cap = 0, int Hkv = 1) {
  int rc = check_common(d, b, dtype, sign_bits);
  if (rc != AXR_OK) return rc;
  if (n < 0) return fail(AXR_EINVAL, "n=%lld is negative", static_cast<long long>(n));
  if (n == 0) return ok();
  if (x == nullptr) return fail(AXR_EINVAL, "input pointer is null");
  if (!aligned(x, 16)) return fail(AXR_EALIGN, "input must be 16-byte aligned");
  if (mode == axr::kWriteQuantize) {
    if (packed == nullptr || norms == nullptr)
      return fail(AXR_EINVAL, "packed and norms must be non-null");
    if (!aligned(packed, 16)) return fail(AXR_EALIGN, "packed must be 16-byte aligned");
    if (!aligned(norms, 4)) return fail(AXR_EALIGN, "norms must be 4-byte aligned");
  } else {
    if (y == nullptr) return fail(AXR_EINVAL, "y is null");
    if (!aligned(y, 16)) return fail(AXR_EALIGN, "y must be 16-byte aligned");
  }
  axr::WriteParams p;
  std::memset(&p, 0, sizeof(p));
  fill_signs(p.sign, sign_bits, d);
  const axr::Codebook& cb = axr::cached_codebook(d, b);
  const int half = 1 << (b - 1);
  const double sqrt_d = std::sqrt(static_cast<double>(d));
  for (int i = 0; i + 1 < half; ++i) p.tpos[i] = static_cast<float>(cb.threshold[half + i] * sqrt_d);
  p.inv_sqrt_d = static_cast<float>(1.0 / sqrt_d);
  p.pos = pos;
  p.t_cap = t_cap;
  p.Hkv = Hkv;
  int err = axr::launch_write(x, dtype, n, d, b, p, packed, norms, y, mode, stream);
  return hip_status(err, "write kernel launch");
}

int axr_quantize_keys(const void* keys, int dtype, int64_t n, int d, int b,
                      const uint32_t* sign_bits, uint32_t* packed, float* norms, void* stream) {
  return write_common(keys, dtype, n, d, b, sign_bits, packed, norms, nullptr,
                      axr::kWriteQuantize, stream);
}

int axr_transform(const void* x, int dtype, int64_t n, int d, const uint32_t* sign_bits,
                  int normalize, float* y, void* stream) {
  // b only selects a kernel instance here; the transform does not depend on it.
  return write_common(x, dtype, n, d, 3, sign_bits, nullptr, nullptr, y,
                      normalize ? axr::kWriteTransformNormalized : axr::kWriteTransform, stream);
}

int axr_append_keys(const void* keys, int dtype, int B, int Hkv, int d, int b,
                    const uint32_t* sign_bits, const int32_t* pos, int64_t t_cap,
                    uint32_t* packed, float* norms, void* stream) {
  if (B < 0 || Hkv < 0) return fail(AXR_EINVAL, "negative size (B=%d Hkv=%d)", B, Hkv);
  if (t_cap < 1) return fail(AXR_EINVAL, "t_cap=%lld must be >= 1", static_cast<long long>(t_cap));
  const int64_t n = static_cast<int64_t>(B) * Hkv;
  if (n > INT32_MAX) return fail(AXR_EUNSUPPORTED, "B*Hkv=%lld exceeds 2^31-1",
                                 static_cast<long long>(n));
  if (n > 0 && pos == nullptr) return fail(AXR_EINVAL, "pos is null");
  if (n > 0 && !aligned(pos, 4)) return fail(AXR_EALIGN, "pos must be 4-byte aligned");
  return write_common(keys, dtype, n, d, b, sign_bits, packed, norms, nullptr,
                      axr::kWriteQuantize, stream, pos, t_cap, Hkv > 0 ? Hkv : 1);
}

// Validates the sizes shared by every read-path call.
static int check_score_sizes(int d, int b, int q_dtype, const uint32_t* sign_bits, int B, int Hq,
                             int Hkv, int64_t T, int64_t t_cap) {
  int rc = check_common(d, b, q_dtype, sign_bits);
  if (rc != AXR_OK) return rc;
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0)
    return fail(AXR_EINVAL, "negative size (B=%d Hq=%d Hkv=%d T=%lld)", B, Hq, Hkv,
                static_cast<long long>(T));
  if (Hkv == 0 || Hq == 0) return fail(AXR_EINVAL, "Hq and Hkv must be positive");
  if (Hq % Hkv != 0) return fail(AXR_EINVAL, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (t_cap < T) return fail(AXR_EINVAL, "t_cap=%lld is smaller than T=%lld",
                             static_cast<long long>(t_cap), static_cast<long long>(T));
  if (Hq / Hkv > 64) return fail(AXR_EUNSUPPORTED, "Hq/Hkv=%d exceeds 64", Hq / Hkv);
  // one (batch, KV head) row of records is addressed with 32-bit offsets
  if (T > 0 && T * static_cast<int64_t>(d) * b / 8 > INT32_MAX)
    return fail(AXR_EUNSUPPORTED, "T=%lld tokens exceed 2 GiB of records per row",
                static_cast<long long>(T));
  return AXR_OK;
}

// Score-kernel parameters for validated sizes (everything but the tiling).
static axr::ScoreParams score_params(const uint32_t* sign_bits, int Hq, int Hkv, int64_t T,
                                     int64_t t_cap, int d, int b, const int32_t* lens) {
  axr::ScoreParams p;
  std::memset(&p, 0, sizeof(p));
  fill_signs(p.sign, sign_bits, d);
  const axr::Codebook& cb = axr::cached_codebook(d, b);
  for (int i = 0; i < (1 << b); ++i) p.centroid[i] = static_cast<float>(cb.centroid[i]);
  p.T = T;
  p.t_cap = t_cap;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.lens = lens;
  return p;
}

static int score_common(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                        const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                        int64_t T, int64_t t_cap, int d, int b, float* scores, void* stream) {
  int rc = check_score_sizes(d, b, q_dtype, sign_bits, B, Hq, Hkv, T, t_cap);
  if (rc != AXR_OK) return rc;
  if (B == 0 || T == 0) return ok();
  if (q == nullptr || packed == nullptr || norms == nullptr || scores == nullptr)
    return fail(AXR_EINVAL, "q, packed, norms and scores must be non-null");
  if (!aligned(q, 16)) return fail(AXR_EALIGN, "q must be 16-byte aligned");
  if (!aligned(packed, 16)) return fail(AXR_EALIGN, "packed must be 16-byte aligned");
  if (!aligned(norms, 4) || !aligned(scores, 4))
    return fail(AXR_EALIGN, "norms and scores must be 4-byte aligned");
  const axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, t_cap, d, b, lens);
  int err = axr::launch_score(q, q_dtype, packed, norms, B, d, b, p, scores, stream);
  return hip_status(err, "score kernel launch");
}

// Tiles per score row for these sizes (sizes already validated).
static int score_tiles(const uint32_t* sign_bits, int B, int Hq, int Hkv, int64_t T,
                       int64_t t_cap, int d, int b, axr::ScoreParams* plan) {
  const axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, t_cap, d, b, nullptr);
  return axr::launch_score(nullptr, AXR_F32, nullptr, nullptr, B, d, b, p, nullptr, nullptr,
                           plan);
}

int axr_score(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
              const uint32_t* sign_bits, int B, int Hq, int Hkv, int64_t T, int64_t t_cap,
              int d, int b, float* scores, void* stream) {
  return score_common(q, q_dtype, packed, norms, sign_bits, B, Hq, Hkv, nullptr, T, t_cap, d, b,
                      scores, stream);
}

int axr_score_softmax_workspace(int B, int Hq, int Hkv, int64_t T, int d, int b,
                                int64_t* bytes) {
  if (bytes == nullptr) return fail(AXR_EINVAL, "bytes is null");
  static const uint32_t zero_signs[axr::kMaxSignWords] = {};
  int rc = check_score_sizes(d, b, AXR_F32, zero_signs, B, Hq, Hkv, T, T);
  if (rc != AXR_OK) return rc;
  if (B == 0 || T == 0) {
    *bytes = 0;
    return ok();
  }
  axr::ScoreParams plan;
  int err = score_tiles(zero_signs, B, Hq, Hkv, T, T, d, b, &plan);
  if (err != 0) return fail(AXR_EUNSUPPORTED, "no launch configuration for these sizes");
  *bytes = static_cast<int64_t>(B) * Hq * plan.tiles * 2 * static_cast<int64_t>(sizeof(float));
  return ok();
}

int axr_score_softmax(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                      const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                      int64_t T, int64_t t_cap, int d, int b, float scale, float* probs,
                      float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  int rc = check_score_sizes(d, b, q_dtype, sign_bits, B, Hq, Hkv, T, t_cap);
  if (rc != AXR_OK) return rc;
  if (!std::isfinite(scale)) return fail(AXR_EINVAL, "scale must be finite");
  if (B == 0 || T == 0) return ok();
  if (q == nullptr || packed == nullptr || norms == nullptr || probs == nullptr)
    return fail(AXR_EINVAL, "q, packed, norms and probs must be non-null");
  if (workspace == nullptr) return fail(AXR_EINVAL, "workspace is null");
  if (!aligned(q, 16)) return fail(AXR_EALIGN, "q must be 16-byte aligned");
  if (!aligned(packed, 16)) return fail(AXR_EALIGN, "packed must be 16-byte aligned");
  if (!aligned(norms, 4) || !aligned(probs, 4) || (lse != nullptr && !aligned(lse, 4)) ||
      (lens != nullptr && !aligned(lens, 4)))
    return fail(AXR_EALIGN, "norms, probs, lse and lens must be 4-byte aligned");
  if (!aligned(workspace, 8)) return fail(AXR_EALIGN, "workspace must be 8-byte aligned");
  axr::ScoreParams plan;
  if (score_tiles(sign_bits, B, Hq, Hkv, T, t_cap, d, b, &plan) != 0)
    return fail(AXR_EUNSUPPORTED, "no launch configuration for these sizes");
  const int64_t need = static_cast<int64_t>(B) * Hq * plan.tiles * 2 * 4;
  if (workspace_bytes < need)
    return fail(AXR_EINVAL, "workspace of %lld bytes is smaller than the %lld required",
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
  axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, t_cap, d, b, lens);
  p.partials = static_cast<float*>(workspace);
  p.scale = scale;
  int err = axr::launch_score(q, q_dtype, packed, norms, B, d, b, p, probs, stream);
  if (err != 0) return hip_status(err, "score kernel launch");
  err = axr::launch_softmax(probs, p.partials, lens, B, Hq, T, plan.tiles, plan.tile_len, scale,
                            lse, stream);
  return hip_status(err, "softmax kernel launch");
}

int axr_score_ragged(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                     const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                     int64_t T, int64_t t_cap, int d, int b, float* scores, void* stream) {
  if (B > 0 && T > 0) {
    if (lens == nullptr) return fail(AXR_EINVAL, "lens is null");
    if (!aligned(lens, 4)) return fail(AXR_EALIGN, "lens must be 4-byte aligned");
  }
  return score_common(q, q_dtype, packed, norms, sign_bits, B, Hq, Hkv, lens, T, t_cap, d, b,
                      scores, stream);
}

}  // extern "C"
