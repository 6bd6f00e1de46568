// Softmax of score rows from split-T partials, for gfx950.
//
// The scores of a (batch, query head) row are produced by several blocks of
// the score kernel, one per tile of tokens; each block leaves the largest
// scaled score of its tile and the sum of exp(scaled score - that maximum).
// Here every block of a row first merges the row's partials (a handful of
// tiles) into the row's (M, L), then turns its chunk of the row into
// probabilities in place: p = exp(scale * s - M) / L.  The kernel streams
// each score once in and once out (HBM-bound).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "axr_device.h"
#include "axr_internal.h"

namespace axr {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int64_t kChunk = static_cast<int64_t>(kThreads) * kPerThread;   // tokens per block

__device__ __forceinline__ void merge(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  if (mm != -INFINITY) {
    l = l * expf(m - mm) + l2 * expf(m2 - mm);
    m = mm;
  }
}

__global__ __launch_bounds__(kThreads) void softmax_rows(float* __restrict__ scores,
                                                        const float* __restrict__ partials,
                                                        const int32_t* __restrict__ lens,
                                                        int Hq, int64_t T, int tiles,
                                                        int64_t chunks, float scale,
                                                        float* __restrict__ lse) {
  const int64_t row = blockIdx.x / chunks;              // bi * Hq + h
  const int64_t c = blockIdx.x % chunks;
  const int bi = static_cast<int>(row / Hq);
  int64_t len = T;
  if (lens != nullptr) {
    const int64_t l = lens[bi];
    len = l < 0 ? 0 : (l < T ? l : T);
  }
  const int64_t t0 = c * kChunk;
  if (t0 >= len) {                                      // block-uniform
    if (c == 0 && lse != nullptr && threadIdx.x == 0) lse[row] = -INFINITY;   // empty row
    return;
  }

  // The chunk's loads go out first, so that their latency overlaps the merge
  // of the partials; all of them before any store (the row is rewritten in
  // place, and the compiler would keep each load behind the previous store).
  float* r = scores + row * T;
  const int64_t t1 = t0 + kChunk < len ? t0 + kChunk : len;
  float v[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t t = t0 + static_cast<int64_t>(k) * kThreads + threadIdx.x;
    v[k] = t < t1 ? r[t] : 0.0f;
  }

  // merge the row's tile partials (wave 0), broadcast through LDS
  __shared__ float ml[2];
  if (threadIdx.x < 64) {
    float m = -INFINITY, l = 0.0f;
    for (int i = threadIdx.x; i < tiles; i += 64) {
      const float* p = partials + (row * tiles + i) * 2;
      merge(m, l, p[0], p[1]);
    }
    merge(m, l, lane_xor<1>(m), lane_xor<1>(l));
    merge(m, l, lane_xor<2>(m), lane_xor<2>(l));
    merge(m, l, lane_xor<4>(m), lane_xor<4>(l));
    merge(m, l, lane_xor<8>(m), lane_xor<8>(l));
    merge(m, l, lane_xor<16>(m), lane_xor<16>(l));
    merge(m, l, lane_xor<32>(m), lane_xor<32>(l));
    if (threadIdx.x == 0) {
      ml[0] = m;
      ml[1] = l;
      if (lse != nullptr && c == 0) lse[row] = m + logf(l);
    }
  }
  __syncthreads();
  const float m = ml[0];
  const float inv_l = 1.0f / ml[1];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int64_t t = t0 + static_cast<int64_t>(k) * kThreads + threadIdx.x;
    // the scaled score rounded as the score kernel rounded it for (m, l)
    if (t < t1) r[t] = expf(mul_rounded(scale, v[k]) - m) * inv_l;
  }
}

}  // namespace

int launch_softmax(float* scores, const float* partials, const int32_t* lens, int B, int Hq,
                   int64_t T, int tiles, int64_t tile_len, float scale, float* lse,
                   void* stream) {
  (void)tile_len;
  const int64_t chunks = (T + kChunk - 1) / kChunk;
  const int64_t grid = static_cast<int64_t>(B) * Hq * chunks;
  if (grid == 0) return 0;
  if (grid > 0x7FFFFFFF) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(softmax_rows, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), scores, partials, lens, Hq, T, tiles,
                     chunks, scale, lse);
  return static_cast<int>(hipGetLastError());
}

}  // namespace axr
