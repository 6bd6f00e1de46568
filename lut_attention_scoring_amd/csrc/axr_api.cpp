// C-ABI layer: argument validation, error reporting, codebook preparation and
// kernel dispatch.  Every check runs before the first HIP call, so rejected
// calls never touch the device.  See include/axr.h for the contract.

#include "axr.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <climits>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

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

// Scale K of the 4-bit quantizer's cell table, in cells per unit of
// z / ||k||.  The kernel compares z with the signed thresholds P_i ||k||
// (P_i = -tpos, 0, +tpos), and |z| <= zmax ||k|| (sqrt(d) for the
// unnormalised Hadamard transform, 1 for the rotations).  K is the smallest
// value, stepping up from one cell per smallest threshold gap (so that no
// cell holds two thresholds), that puts every nonzero P_i K + kCellMid at
// least 0.05 of a cell from a cell boundary, within the table's reach
// (zmax K <= kCellMid - 2).  The kernel's cell position is within ~1e-5 of a
// cell of its exact value, so a z near a cell boundary is never near a
// threshold other than 0, which lies exactly on boundary kCellMid, where
// rounding cannot carry z across.
static float cell_scale(const float* tpos, int half, double zmax) {
  const int nt = 2 * half - 1;
  double P[axr::kMaxLevels - 1];
  for (int j = 0; j + 1 < half; ++j) {
    P[half + j] = tpos[j];
    P[half - 2 - j] = -static_cast<double>(tpos[j]);
  }
  P[half - 1] = 0.0;
  double gap = P[1] - P[0];
  for (int i = 1; i + 1 < nt; ++i) gap = std::min(gap, P[i + 1] - P[i]);
  const double mid = axr::kCellMid;
  const double Kmax = (mid - 2.0) / (zmax * 1.001);
  for (double K = 1.001 / gap; K <= Kmax; K += 1e-4 / gap) {
    const double Kf = static_cast<float>(K);   // the kernel's value
    bool good = true;
    for (int i = 0; i < nt && good; ++i) {
      if (i == half - 1) continue;
      const double t = P[i] * Kf + mid;
      const double f = t - std::floor(t);
      good = f >= 0.05 && f <= 0.95;
    }
    if (good) return static_cast<float>(K);
  }
  return 0.0f;   // no scale found: the kernel keeps its threshold search
}

// cell_scale for (d, b, transform), computed once per process (thread-safe).
static float cached_cell_scale(int d, int b, int tf, const float* tpos, int half, double zmax) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, float> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(d, b, tf);
  auto it = cache.find(key);
  if (it == cache.end()) it = cache.emplace(key, cell_scale(tpos, half, zmax)).first;
  return it->second;
}

// Write-kernel parameters: sign words and the positive thresholds scaled by
// sqrt(d) (the kernel compares against them times the key's norm).
// (The block-quaternion transform is orthonormal as it stands, so there the
// factor is 1.)
static axr::WriteParams write_params(const uint32_t* sign_bits, int d, int b,
                                     int tf = axr::kWht) {
  axr::WriteParams p;
  std::memset(&p, 0, sizeof(p));
  if (sign_bits != nullptr) fill_signs(p.sign, sign_bits, d);
  const axr::Codebook& cb = axr::cached_codebook(d, b);
  const int half = 1 << (b - 1);
  const double sqrt_d = tf == axr::kWht ? std::sqrt(static_cast<double>(d)) : 1.0;
  for (int i = 0; i + 1 < half; ++i) p.tpos[i] = static_cast<float>(cb.threshold[half + i] * sqrt_d);
  p.inv_sqrt_d = static_cast<float>(1.0 / sqrt_d);
  p.cell_k = b == 4 ? cached_cell_scale(d, b, tf, p.tpos, half, tf == axr::kWht ? sqrt_d : 1.0)
                   : 0.0f;
  if (p.cell_k > 0.0f) {
    // positions of the 15 signed thresholds on the cell scale, ascending, in
    // the fp32 arithmetic the kernel compares with
    float pos[axr::kMaxLevels - 1];
    for (int i = 0; i < 15; ++i) {
      const float th = i < 7 ? -p.tpos[6 - i] : (i == 7 ? 0.0f : p.tpos[i - 8]);
      pos[i] = std::fmaf(th, p.cell_k, axr::kCellMid);
    }
    for (int c = 0; c < axr::kCells; ++c) {
      uint32_t cnt = 0;
      while (cnt < 15 && pos[cnt] < static_cast<float>(c)) ++cnt;
      const float nxt = cnt < 15 ? pos[cnt] : INFINITY;
      p.cells[2 * c] = cnt;
      std::memcpy(&p.cells[2 * c + 1], &nxt, 4);
    }
  }
  p.t_cap = 0;
  p.Hkv = 1;
  return p;
}

static int write_common(const void* x, int dtype, int64_t n, int d, int b,
                        const uint32_t* sign_bits, uint32_t* packed, float* norms, float* y,
                        int mode, void* stream, const int32_t* pos = nullptr,
                        int64_t t_cap = 0, int Hkv = 1, int tf = axr::kWht,
                        const float* quats = nullptr) {
  static const uint32_t no_signs[axr::kMaxSignWords] = {};
  int rc = check_common(d, b, dtype, tf == axr::kWht ? sign_bits : no_signs);
  if (rc != AXR_OK) return rc;
  if (tf != axr::kWht && n > 0) {
    if (quats == nullptr) return fail(AXR_EINVAL, "quats is null");
    if (!aligned(quats, 16)) return fail(AXR_EALIGN, "quats must be 16-byte aligned");
  }
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
  axr::WriteParams p = write_params(tf == axr::kWht ? sign_bits : nullptr, d, b, tf);
  p.pos = pos;
  p.t_cap = t_cap;
  p.Hkv = Hkv;
  p.quats = quats;
  int err = axr::launch_write(x, dtype, n, d, b, p, packed, norms, y, mode, stream, tf);
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

int axr_quantize_keys_isoquant(const void* keys, int dtype, int64_t n, int d, int b,
                               const float* quats, int full, uint32_t* packed, float* norms,
                               void* stream) {
  return write_common(keys, dtype, n, d, b, nullptr, packed, norms, nullptr,
                      axr::kWriteQuantize, stream, nullptr, 0, 1,
                      full ? axr::kIsoFull : axr::kIsoFast, quats);
}

int axr_transform_isoquant(const void* x, int dtype, int64_t n, int d, const float* quats,
                           int full, int normalize, float* y, void* stream) {
  return write_common(x, dtype, n, d, 3, nullptr, nullptr, nullptr, y,
                      normalize ? axr::kWriteTransformNormalized : axr::kWriteTransform, stream,
                      nullptr, 0, 1, full ? axr::kIsoFull : axr::kIsoFast, quats);
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
  // (this also bounds the score rows of one block's query heads, addressed
  // the same way: at most 8 heads x 4 B per token, never more than the
  // d*b/8 >= 32 B of a record)
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

// axr_score_softmax, with the split-T partials either in the caller's
// workspace or (use_scratch) in the library's own device array.
static int score_softmax_common(const void* q, int q_dtype, const uint32_t* packed,
                                const float* norms, const uint32_t* sign_bits, int B, int Hq,
                                int Hkv, const int32_t* lens, int64_t T, int64_t t_cap, int d,
                                int b, float scale, float* probs, float* lse, void* workspace,
                                int64_t workspace_bytes, bool use_scratch, void* stream) {
  int rc = check_score_sizes(d, b, q_dtype, sign_bits, B, Hq, Hkv, T, t_cap);
  if (rc != AXR_OK) return rc;
  if (!std::isfinite(scale)) return fail(AXR_EINVAL, "scale must be finite");
  if (B == 0 || T == 0) return ok();
  if (q == nullptr || packed == nullptr || norms == nullptr || probs == nullptr)
    return fail(AXR_EINVAL, "q, packed, norms and probs must be non-null");
  if (!use_scratch && workspace == nullptr) return fail(AXR_EINVAL, "workspace is null");
  if (!aligned(q, 16)) return fail(AXR_EALIGN, "q must be 16-byte aligned");
  if (!aligned(packed, 16)) return fail(AXR_EALIGN, "packed must be 16-byte aligned");
  if (!aligned(norms, 4) || !aligned(probs, 4) || (lse != nullptr && !aligned(lse, 4)) ||
      (lens != nullptr && !aligned(lens, 4)))
    return fail(AXR_EALIGN, "norms, probs, lse and lens must be 4-byte aligned");
  if (!use_scratch && !aligned(workspace, 8))
    return fail(AXR_EALIGN, "workspace must be 8-byte aligned");
  axr::ScoreParams plan;
  if (score_tiles(sign_bits, B, Hq, Hkv, T, t_cap, d, b, &plan) != 0)
    return fail(AXR_EUNSUPPORTED, "no launch configuration for these sizes");
  const int64_t need = static_cast<int64_t>(B) * Hq * plan.tiles * 2 * 4;
  if (use_scratch) {
    if (need > axr::kScratchBytes)
      return fail(AXR_EUNSUPPORTED,
                  "these sizes need %lld bytes of split-T partials, more than the %lld bytes "
                  "of library scratch (use axr_score_softmax with a workspace)",
                  static_cast<long long>(need), static_cast<long long>(axr::kScratchBytes));
    const int err = axr::scratch_address(&workspace);
    if (err != 0) return hip_status(err, "library scratch address");
  } else if (workspace_bytes < need) {
    return fail(AXR_EINVAL, "workspace of %lld bytes is smaller than the %lld required",
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
  }
  axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, t_cap, d, b, lens);
  p.partials = static_cast<float*>(workspace);
  p.scale = scale;
  int err = axr::launch_score(q, q_dtype, packed, norms, B, d, b, p, probs, stream);
  if (err != 0) return hip_status(err, "score kernel launch");
  err = axr::launch_softmax(probs, p.partials, lens, B, Hq, T, plan.tiles, plan.tile_len, scale,
                            lse, stream);
  return hip_status(err, "softmax kernel launch");
}

int axr_score_softmax(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                      const uint32_t* sign_bits, int B, int Hq, int Hkv, const int32_t* lens,
                      int64_t T, int64_t t_cap, int d, int b, float scale, float* probs,
                      float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
  return score_softmax_common(q, q_dtype, packed, norms, sign_bits, B, Hq, Hkv, lens, T, t_cap,
                              d, b, scale, probs, lse, workspace, workspace_bytes, false, stream);
}

int axr_score_softmax_noalloc(const void* q, int q_dtype, const uint32_t* packed,
                              const float* norms, const uint32_t* sign_bits, int B, int Hq,
                              int Hkv, const int32_t* lens, int64_t T, int64_t t_cap, int d,
                              int b, float scale, float* probs, float* lse, void* stream) {
  return score_softmax_common(q, q_dtype, packed, norms, sign_bits, B, Hq, Hkv, lens, T, t_cap,
                              d, b, scale, probs, lse, nullptr, 0, true, stream);
}

// Workspace layout of the sign-pattern selection (offsets 256-byte aligned):
// exact scores, table scores (fp32 [S*B][Hq][T] each), records and norms of
// the calibration keys.
struct SelectLayout {
  int64_t exact, lut, packed, norms, partials, total;
};

static SelectLayout select_layout(int S, int B, int Hq, int Hkv, int64_t T, int d, int b) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t rows = static_cast<int64_t>(S) * B;
  const int64_t n_scores = rows * Hq * T, n_keys = rows * Hkv * T;
  SelectLayout l;
  l.exact = 0;
  l.lut = up(l.exact + n_scores * 4);
  l.packed = up(l.lut + n_scores * 4);
  l.norms = up(l.packed + n_keys * (static_cast<int64_t>(d) * b / 8));
  l.partials = up(l.norms + n_keys * 4);
  l.total = up(l.partials + static_cast<int64_t>(axr::score_error_partials(S)) * 8);
  return l;
}

static int check_select_sizes(int S, int B, int Hq, int Hkv, int64_t T, int d, int b,
                              int dtype, int q_dtype) {
  static const uint32_t zero_signs[axr::kMaxSignWords] = {};
  if (S < 0) return fail(AXR_EINVAL, "S=%d is negative", S);
  if (S > 64) return fail(AXR_EUNSUPPORTED, "S=%d calibration samples exceed 64", S);
  int rc = check_score_sizes(d, b, q_dtype, zero_signs, B, Hq, Hkv, T, T);
  if (rc != AXR_OK) return rc;
  if (!supported_dtype(dtype)) return fail(AXR_EUNSUPPORTED, "dtype=%d is not supported", dtype);
  if (static_cast<int64_t>(S) * B > INT32_MAX / 2)
    return fail(AXR_EUNSUPPORTED, "S*B=%lld is too large", static_cast<long long>(S) * B);
  return AXR_OK;
}

int axr_sign_selection_workspace(int S, int B, int Hq, int Hkv, int64_t T, int d, int b,
                                 int64_t* bytes) {
  if (bytes == nullptr) return fail(AXR_EINVAL, "bytes is null");
  int rc = check_select_sizes(S, B, Hq, Hkv, T, d, b, AXR_F32, AXR_F32);
  if (rc != AXR_OK) return rc;
  *bytes = select_layout(S, B, Hq, Hkv, T, d, b).total;
  return ok();
}

int axr_sign_selection_errors(const void* keys, int dtype, const void* q, int q_dtype, int S,
                              int B, int Hq, int Hkv, int64_t T, int d, int b,
                              const uint32_t* candidates, int C, double* errors,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  int rc = check_select_sizes(S, B, Hq, Hkv, T, d, b, dtype, q_dtype);
  if (rc != AXR_OK) return rc;
  if (C < 0) return fail(AXR_EINVAL, "C=%d is negative", C);
  if (C == 0 || S == 0 || B == 0 || T == 0) return ok();
  if (candidates == nullptr) return fail(AXR_EINVAL, "candidates is null");
  if (keys == nullptr || q == nullptr || errors == nullptr || workspace == nullptr)
    return fail(AXR_EINVAL, "keys, q, errors and workspace must be non-null");
  if (!aligned(keys, 16) || !aligned(q, 16)) return fail(AXR_EALIGN, "keys and q must be 16-byte aligned");
  if (!aligned(errors, 8)) return fail(AXR_EALIGN, "errors must be 8-byte aligned");
  if (!aligned(workspace, 256)) return fail(AXR_EALIGN, "workspace must be 256-byte aligned");
  const SelectLayout lay = select_layout(S, B, Hq, Hkv, T, d, b);
  if (workspace_bytes < lay.total)
    return fail(AXR_EINVAL, "workspace of %lld bytes is smaller than the %lld required",
                static_cast<long long>(workspace_bytes), static_cast<long long>(lay.total));
  char* ws = static_cast<char*>(workspace);
  float* exact = reinterpret_cast<float*>(ws + lay.exact);
  float* lut = reinterpret_cast<float*>(ws + lay.lut);
  uint32_t* packed = reinterpret_cast<uint32_t*>(ws + lay.packed);
  float* norms = reinterpret_cast<float*>(ws + lay.norms);
  double* partials = reinterpret_cast<double*>(ws + lay.partials);
  const int rows = S * B;
  const int64_t n = static_cast<int64_t>(rows) * Hkv * T;
  int err = axr::launch_dense_scores(keys, dtype, q, q_dtype, rows, Hq, Hkv, T, d, exact, stream);
  if (err != 0) return hip_status(err, "exact-score kernel launch");
  const int words = d / 32;
  for (int c = 0; c < C; ++c) {
    const uint32_t* sc = candidates + static_cast<size_t>(c) * words;
    const axr::WriteParams wp = write_params(sc, d, b);
    err = axr::launch_write(keys, dtype, n, d, b, wp, packed, norms, nullptr, axr::kWriteQuantize,
                            stream);
    if (err != 0) return hip_status(err, "write kernel launch");
    const axr::ScoreParams sp = score_params(sc, Hq, Hkv, T, T, d, b, nullptr);
    err = axr::launch_score(q, q_dtype, packed, norms, rows, d, b, sp, lut, stream);
    if (err != 0) return hip_status(err, "score kernel launch");
    err = axr::launch_score_error(lut, exact, S, static_cast<int64_t>(B) * Hq * T, partials,
                                  errors + static_cast<size_t>(c) * S * 2, stream);
    if (err != 0) return hip_status(err, "error kernel launch");
  }
  return ok();
}

int axr_sign_selection_choose(const double* errors, int C, int S, int* index,
                              double* objective) {
  if (C < 1 || S < 1) return fail(AXR_EINVAL, "C=%d and S=%d must be positive", C, S);
  if (errors == nullptr || index == nullptr)
    return fail(AXR_EINVAL, "errors and index must be non-null");
  const int64_t n = static_cast<int64_t>(C) * S * 2;
  for (int64_t i = 0; i < n; ++i) {
    if (!(errors[i] >= 0.0))
      return fail(AXR_EINVAL, "error sum %lld is negative or NaN", static_cast<long long>(i));
  }
  int best = 0;
  double best_obj = 0.0;
  for (int c = 0; c < C; ++c) {
    double worst = 0.0;
    for (int i = 0; i < S; ++i) {
      const double err = errors[(static_cast<int64_t>(c) * S + i) * 2];
      const double ref = errors[(static_cast<int64_t>(c) * S + i) * 2 + 1];
      const double r = ref > 0.0 ? std::sqrt(err / ref) : (err > 0.0 ? HUGE_VAL : 0.0);
      worst = std::max(worst, r);
    }
    if (objective != nullptr) objective[c] = worst;
    if (c == 0 || worst < best_obj) {
      best = c;
      best_obj = worst;
    }
  }
  *index = best;
  return ok();
}

int axr_decode_step(const void* q, int q_dtype, const void* k_new, int k_dtype,
                    const uint32_t* sign_bits, const int32_t* pos, int B, int Hq, int Hkv,
                    int64_t T, int64_t t_cap, int d, int b, uint32_t* packed, float* norms,
                    float* scores, void* stream) {
  int rc = check_score_sizes(d, b, q_dtype, sign_bits, B, Hq, Hkv, T, t_cap);
  if (rc != AXR_OK) return rc;
  if (!supported_dtype(k_dtype)) return fail(AXR_EUNSUPPORTED, "k_dtype=%d is not supported", k_dtype);
  if (B == 0) return ok();
  if (T == 0) {                                 // nothing to score: the append alone
    if (t_cap == 0) return ok();
    return axr_append_keys(k_new, k_dtype, B, Hkv, d, b, sign_bits, pos, t_cap, packed, norms,
                           stream);
  }
  if (q == nullptr || k_new == nullptr || pos == nullptr || packed == nullptr ||
      norms == nullptr || scores == nullptr)
    return fail(AXR_EINVAL, "q, k_new, pos, packed, norms and scores must be non-null");
  if (!aligned(q, 16) || !aligned(packed, 16))
    return fail(AXR_EALIGN, "q and packed must be 16-byte aligned");
  if (!aligned(k_new, 4) || !aligned(pos, 4) || !aligned(norms, 4) || !aligned(scores, 4))
    return fail(AXR_EALIGN, "k_new, pos, norms and scores must be 4-byte aligned");
  axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, t_cap, d, b, nullptr);
  p.knew = k_new;
  p.kdt = k_dtype;
  p.pos = pos;
  p.packed_out = packed;
  p.norms_out = norms;
  const axr::WriteParams wp = write_params(sign_bits, d, b);
  for (int i = 0; i < axr::kMaxLevels / 2; ++i) p.tpos[i] = wp.tpos[i];
  int err = axr::launch_score(q, q_dtype, packed, norms, B, d, b, p, scores, stream);
  return hip_status(err, "score kernel launch");
}

int axr_quantize_score(const void* keys, int k_dtype, const void* q, int q_dtype,
                       const uint32_t* sign_bits, int B, int Hq, int Hkv, int64_t T, int d,
                       int b, uint32_t* packed, float* norms, float* scores, void* stream) {
  int rc = check_score_sizes(d, b, q_dtype, sign_bits, B, Hq, Hkv, T, T);
  if (rc != AXR_OK) return rc;
  if (!supported_dtype(k_dtype)) return fail(AXR_EUNSUPPORTED, "k_dtype=%d is not supported", k_dtype);
  if (d != 128 || b > 3)
    return fail(AXR_EUNSUPPORTED, "quantize-and-score is built for d=128 and b=2 or 3 (d=%d b=%d)",
                d, b);
  // every key is quantized by one block: G <= 4 (one table), or G = 8 at
  // b = 3 (two tables of four heads in one block)
  const int G = Hq / Hkv;
  if (G > 4 && !(G == 8 && b == 3))
    return fail(AXR_EUNSUPPORTED, "quantize-and-score needs Hq/Hkv <= 4, or 8 at b=3 (got %d, b=%d)",
                G, b);
  // one row of raw keys is addressed with 32-bit offsets
  const int64_t esize = k_dtype == AXR_F32 ? 4 : 2;
  if (T > 0 && T * d * esize > INT32_MAX)
    return fail(AXR_EUNSUPPORTED, "T=%lld tokens exceed 2 GiB of keys per row",
                static_cast<long long>(T));
  if (B == 0 || T == 0) return ok();
  if (keys == nullptr || q == nullptr || packed == nullptr || norms == nullptr ||
      scores == nullptr)
    return fail(AXR_EINVAL, "keys, q, packed, norms and scores must be non-null");
  if (!aligned(keys, 16) || !aligned(q, 16) || !aligned(packed, 16))
    return fail(AXR_EALIGN, "keys, q and packed must be 16-byte aligned");
  if (!aligned(norms, 4) || !aligned(scores, 4))
    return fail(AXR_EALIGN, "norms and scores must be 4-byte aligned");
  axr::ScoreParams p = score_params(sign_bits, Hq, Hkv, T, T, d, b, nullptr);
  const axr::WriteParams wp = write_params(sign_bits, d, b);
  for (int i = 0; i < axr::kMaxLevels / 2; ++i) p.tpos[i] = wp.tpos[i];
  p.inv_sqrt_d = wp.inv_sqrt_d;
  p.keys = keys;
  p.kdt = k_dtype;
  p.packed_out = packed;
  p.norms_out = norms;
  int err = axr::launch_score(q, q_dtype, packed, norms, B, d, b, p, scores, stream);
  return hip_status(err, "quantize-and-score kernel launch");
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
