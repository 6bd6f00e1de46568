// Kernels of the one-time sign-pattern selection, for gfx950.
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// the sign pattern is chosen once, without gradients, among a few hundred
// candidates on a few calibration samples.  For every candidate the host
// runs the write and score kernels on the calibration keys; the kernels here
// supply the exact scores to compare with and the per-sample error sums (in
// two fixed-order fp64 passes):
//   err[c][i] = sum (s_lut - s_exact)^2,  ref[c][i] = sum s_exact^2.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "axr.h"
#include "axr_internal.h"

namespace axr {
namespace {

constexpr int kDenseThreads = 256;
constexpr int kMaxGroup = 64;

__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  if (dtype == AXR_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if (dtype == AXR_F16) return __half2float(__ushort_as_half(h));
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Exact fp32 scores q_h . k_t for the G query heads of one (row, KV head):
// one thread per token reads its key once; the G queries sit in LDS.
// Grid: rows * Hkv * ceil(T / kDenseThreads) blocks.
template <int D>
__global__ __launch_bounds__(kDenseThreads) void dense_scores_kernel(
    const void* __restrict__ keys, int kdt, const void* __restrict__ q, int qdt, int Hq,
    int Hkv, int64_t T, int64_t tiles, float* __restrict__ out) {
  const int G = Hq / Hkv;
  const int64_t rk = blockIdx.x / tiles;                 // row * Hkv + kvh
  const int64_t tile = blockIdx.x % tiles;
  const int64_t row = rk / Hkv;
  const int kvh = static_cast<int>(rk % Hkv);
  __shared__ float qs[kMaxGroup * D];
  for (int i = threadIdx.x; i < G * D; i += kDenseThreads) {
    const int g = i / D, j = i % D;
    qs[i] = load_elem(q, qdt, (static_cast<size_t>(row) * Hq + kvh * G + g) * D + j);
  }
  __syncthreads();
  const int64_t t = tile * kDenseThreads + threadIdx.x;
  if (t >= T) return;
  const size_t kbase = (static_cast<size_t>(rk) * T + t) * D;
  for (int g0 = 0; g0 < G; g0 += 8) {
    float acc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) acc[g] = 0.0f;
    for (int j = 0; j < D; ++j) {
      const float k = load_elem(keys, kdt, kbase + j);
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g0 + g < G) acc[g] = fmaf(qs[(g0 + g) * D + j], k, acc[g]);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g0 + g < G) out[(static_cast<size_t>(row) * Hq + kvh * G + g0 + g) * T + t] = acc[g];
  }
}

constexpr int kErrThreads = 256;
constexpr int kErrBlocks = 64;   // blocks per calibration sample

// Block (i, j) sums (lut - exact)^2 and exact^2 over slice j of sample i's
// `per` scores in fp64 and reduces them in a fixed order; the second kernel
// adds the kErrBlocks partials of each sample in order, so the sums do not
// depend on scheduling.
__global__ __launch_bounds__(kErrThreads) void score_error_partial(
    const float* __restrict__ lut, const float* __restrict__ exact, int64_t per,
    double* __restrict__ part) {
  const int sample = blockIdx.x / kErrBlocks;
  const int slice = blockIdx.x % kErrBlocks;
  const int64_t chunk = (per + kErrBlocks - 1) / kErrBlocks;
  const int64_t i0 = slice * chunk;
  const int64_t i1 = i0 + chunk < per ? i0 + chunk : per;
  const size_t base = static_cast<size_t>(sample) * per;
  double e = 0.0, r = 0.0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kErrThreads) {
    const double x = exact[base + i];
    const double dlt = static_cast<double>(lut[base + i]) - x;
    e = fma(dlt, dlt, e);
    r = fma(x, x, r);
  }
  __shared__ double se[kErrThreads], sr[kErrThreads];
  se[threadIdx.x] = e;
  sr[threadIdx.x] = r;
  __syncthreads();
  for (int s = kErrThreads / 2; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) {
      se[threadIdx.x] += se[threadIdx.x + s];
      sr[threadIdx.x] += sr[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = se[0];
    part[2 * blockIdx.x + 1] = sr[0];
  }
}

__global__ __launch_bounds__(64) void score_error_final(const double* __restrict__ part,
                                                       int samples, double* __restrict__ err) {
  const int i = threadIdx.x;
  if (i >= samples) return;
  double e = 0.0, r = 0.0;
  for (int j = 0; j < kErrBlocks; ++j) {
    e += part[2 * (i * kErrBlocks + j)];
    r += part[2 * (i * kErrBlocks + j) + 1];
  }
  err[2 * i] = e;
  err[2 * i + 1] = r;
}

}  // namespace

int launch_dense_scores(const void* keys, int kdt, const void* q, int qdt, int rows, int Hq,
                        int Hkv, int64_t T, int d, float* out, void* stream) {
  const int64_t tiles = (T + kDenseThreads - 1) / kDenseThreads;
  const int64_t grid = static_cast<int64_t>(rows) * Hkv * tiles;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF || Hq / Hkv > kMaxGroup)
    return static_cast<int>(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(grid)), b(kDenseThreads);
  switch (d) {
    case 128: hipLaunchKernelGGL(dense_scores_kernel<128>, g, b, 0, s, keys, kdt, q, qdt, Hq, Hkv, T, tiles, out); break;
    case 256: hipLaunchKernelGGL(dense_scores_kernel<256>, g, b, 0, s, keys, kdt, q, qdt, Hq, Hkv, T, tiles, out); break;
    default: hipLaunchKernelGGL(dense_scores_kernel<512>, g, b, 0, s, keys, kdt, q, qdt, Hq, Hkv, T, tiles, out); break;
  }
  return static_cast<int>(hipGetLastError());
}

int score_error_partials(int samples) { return samples * kErrBlocks * 2; }

int launch_score_error(const float* lut, const float* exact, int samples, int64_t per,
                       double* part, double* err, void* stream) {
  if (samples == 0) return 0;
  if (samples > 64) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(score_error_partial, dim3(samples * kErrBlocks), dim3(kErrThreads), 0, s,
                     lut, exact, per, part);
  hipLaunchKernelGGL(score_error_final, dim3(1), dim3(64), 0, s, part, samples, err);
  return static_cast<int>(hipGetLastError());
}

}  // namespace axr
