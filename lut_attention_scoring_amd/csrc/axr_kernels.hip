// HIP kernels for gfx950 (MI355X): the AXELRAM write path (normalise, sign
// pattern, Walsh-Hadamard transform, Lloyd-Max bucketize, bit-pack) and read
// path (query transform, lookup table in LDS, table-lookup accumulate).
//
// Method: "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638),
// Abstract -- orthogonal transform on write, design-time codebook fixed by
// (d, b), table lookup on read with no inverse transform.
//
// Both kernels stream HBM.  Neither is a dense contraction, so no MFMA is
// used: the write kernel is bound by VALU work per key (butterflies and
// compares), the read kernel by HBM bytes with LDS lookups as the second
// limit.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "axr.h"
#include "axr_internal.h"

namespace axr {
namespace {

constexpr int kBlock = 256;

// ---------------------------------------------------------------------------
// Lane exchange inside aligned groups of up to 16 lanes: returns the value
// held by lane (lane ^ M).  xor 1 and xor 2 are DPP quad permutations, xor 8
// is a DPP rotate by 8 inside a 16-lane row, xor 4 uses ds_swizzle's bitmask
// mode (no DPP control swaps lanes at distance 4).
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int iv = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  } else if constexpr (M == 4) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(iv, (4 << 10) | 0x1F));
  } else {
    static_assert(M == 8, "lane distance must be 1, 2, 4 or 8");
    return __int_as_float(__builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, false));  // row_ror:8
  }
}

// Sum over the aligned group of LPK lanes; every lane gets the same bits.
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPK >= 2) v += lane_xor<1>(v);
  if constexpr (LPK >= 4) v += lane_xor<2>(v);
  if constexpr (LPK >= 8) v += lane_xor<4>(v);
  if constexpr (LPK >= 16) v += lane_xor<8>(v);
  return v;
}

// One Walsh-Hadamard butterfly stage across lanes at distance M: the lane
// with bit M clear keeps a + b, its partner keeps a - b.
template <int M>
__device__ __forceinline__ void lane_stage(float (&x)[32], int lane_in_key) {
  const float sgn = (lane_in_key & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const float p = lane_xor<M>(x[r]);
    x[r] = fmaf(x[r], sgn, p);  // clear: x + p ; set: p - x
  }
}

// ---------------------------------------------------------------------------
// Input loads: 32 consecutive elements of a key, converted to fp32.
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void load32(const void* __restrict__ base, size_t off, float (&x)[32]) {
  if constexpr (DT == AXR_F32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = src[i];
      x[4 * i + 0] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (DT == AXR_F16) {
          x[8 * i + 2 * k] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[k] & 0xFFFFu)));
          x[8 * i + 2 * k + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[k] >> 16)));
        } else {
          x[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
          x[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
      }
    }
  }
}

// Cell index of a transformed coordinate z against thresholds scaled to z's
// units.  P holds the positive thresholds (2^(b-1) - 1 of them, ascending);
// the codebook is symmetric with 0 as its middle threshold.  Counts
// thresholds strictly below |z| by binary search, then mirrors for z <= 0.
template <int BITS>
__device__ __forceinline__ uint32_t bucket(float z, const float (&P)[8]) {
  constexpr uint32_t HALF = 1u << (BITS - 1);
  const float a = fabsf(z);
  uint32_t m;
  if constexpr (BITS == 2) {
    m = a > P[0] ? 1u : 0u;
  } else if constexpr (BITS == 3) {
    const bool c1 = a > P[1];
    const float t = c1 ? P[2] : P[0];
    m = (c1 ? 2u : 0u) + (a > t ? 1u : 0u);
  } else {
    static_assert(BITS == 4, "b must be 2, 3 or 4");
    const bool c1 = a > P[3];
    const float t2 = c1 ? P[5] : P[1];
    const bool c2 = a > t2;
    const float t3 = c1 ? (c2 ? P[6] : P[4]) : (c2 ? P[2] : P[0]);
    m = (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (a > t3 ? 1u : 0u);
  }
  return z > 0.0f ? HALF + m : HALF - 1u - m;
}

// ---------------------------------------------------------------------------
// Write kernel.  A key of D coordinates is held by LPK = D/32 adjacent lanes,
// lane l owning coordinates [32 l, 32 l + 32) in registers.  The transform is
// five butterfly stages inside each lane and log2(LPK) stages across lanes.
// The 32 indices of a lane are exactly BITS words of the packed record, so
// each lane stores its words directly and a wave writes a contiguous span.
// ---------------------------------------------------------------------------
template <int D, int BITS, int DT>
__global__ __launch_bounds__(kBlock) void write_kernel(const void* __restrict__ keys, int64_t n,
                                                     WriteParams prm,
                                                     uint32_t* __restrict__ packed,
                                                     float* __restrict__ norms,
                                                     float* __restrict__ yout, int mode) {
  constexpr int LPK = D / 32;
  constexpr int KPB = kBlock / LPK;
  constexpr int W = D * BITS / 32;
  const int lane_in_key = threadIdx.x % LPK;
  const int key_in_block = threadIdx.x / LPK;
  const uint32_t sw = prm.sign[lane_in_key];
  float P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = prm.tpos[i];

  for (int64_t base = static_cast<int64_t>(blockIdx.x) * KPB; base < n;
       base += static_cast<int64_t>(gridDim.x) * KPB) {
    const int64_t key = base + key_in_block;
    const bool valid = key < n;
    const int64_t kc = valid ? key : n - 1;
    float x[32];
    load32<DT>(keys, static_cast<size_t>(kc) * D + static_cast<size_t>(lane_in_key) * 32, x);

    float ss = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) ss = fmaf(x[r], x[r], ss);
    ss = group_sum<LPK>(ss);
    const float nrm = sqrtf(ss);

#pragma unroll
    for (int r = 0; r < 32; ++r)
      x[r] = __uint_as_float(__float_as_uint(x[r]) ^ (((sw >> r) & 1u) << 31));

#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
      }
    }
    if constexpr (LPK >= 2) lane_stage<1>(x, lane_in_key);
    if constexpr (LPK >= 4) lane_stage<2>(x, lane_in_key);
    if constexpr (LPK >= 8) lane_stage<4>(x, lane_in_key);
    if constexpr (LPK >= 16) lane_stage<8>(x, lane_in_key);

    if (mode == kWriteQuantize) {
      // z = sqrt(d) ||k|| y, so compare z against t sqrt(d) ||k||.
      float S[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) S[i] = P[i] * nrm;
      uint32_t words[BITS];
#pragma unroll
      for (int i = 0; i < BITS; ++i) words[i] = 0u;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const uint32_t v = bucket<BITS>(x[r], S);
        const int pos = r * BITS, wi = pos >> 5, sh = pos & 31;
        words[wi] |= v << sh;
        if (sh + BITS > 32) words[wi + 1] |= v >> (32 - sh);
      }
      if (valid) {
        uint32_t* dst = packed + static_cast<size_t>(key) * W + lane_in_key * BITS;
        if constexpr (BITS == 2) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else if constexpr (BITS == 4) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        } else {
#pragma unroll
          for (int i = 0; i < BITS; ++i) dst[i] = words[i];
        }
        if (lane_in_key == 0) norms[key] = nrm;
      }
    } else {
      float scale = prm.inv_sqrt_d;
      if (mode == kWriteTransformNormalized) scale = nrm > 0.0f ? prm.inv_sqrt_d / nrm : 0.0f;
      if (valid) {
        float4* dst = reinterpret_cast<float4*>(yout + static_cast<size_t>(key) * D +
                                                static_cast<size_t>(lane_in_key) * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          dst[i] = make_float4(x[4 * i] * scale, x[4 * i + 1] * scale, x[4 * i + 2] * scale,
                               x[4 * i + 3] * scale);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Score kernel.  One block serves GB query heads of one (batch, KV head) row
// over one tile of tokens.
//   prologue: q' = H (s * q) / sqrt(d) in LDS; per head a power-of-two
//             fixed-point scale 2^e with sum_j |q'_j| max|c| 2^e < 2^30; the
//             table of P-coordinate groups  LUT[grp][field][g] =
//             round(2^e * sum_{u<P} q'_{P grp + u} c[field_u])  in LDS as int32;
//   loop:     one thread per key: read the packed record and the norm, add one
//             table entry per group (exact int32 sums), scale by 2^-e and by
//             the key's norm, store fp32 scores.
// A P = 2 field is just 2*BITS consecutive record bits, so no reshuffling of
// the stored indices is needed.
// ---------------------------------------------------------------------------
template <int D, int BITS, int GB, int P>
__global__ __launch_bounds__(kBlock) void score_kernel(const void* __restrict__ q, int qdt,
                                                     const uint32_t* __restrict__ packed,
                                                     const float* __restrict__ norms,
                                                     float* __restrict__ scores, ScoreParams prm) {
  constexpr int W = D * BITS / 32;
  constexpr int FB = P * BITS;
  constexpr int NE = 1 << FB;
  constexpr int NG = D / P;
  constexpr uint32_t FMASK = (1u << FB) - 1u;
  extern __shared__ int4 lut_raw[];
  int* lut = reinterpret_cast<int*>(lut_raw);
  __shared__ float qs[GB][D];
  __shared__ float cent[16];
  __shared__ float hscale[GB], hinv[GB];

  const int tid = threadIdx.x;
  const int tile = blockIdx.x % prm.tiles;
  const int hg = (blockIdx.x / prm.tiles) % prm.head_groups;
  const int row = blockIdx.x / (prm.tiles * prm.head_groups);
  const int bi = row / prm.Hkv;
  const int kvh = row % prm.Hkv;
  const int h0 = kvh * prm.G + hg * GB;

  // 1. queries with the sign pattern applied
  for (int i = tid; i < GB * D; i += kBlock) {
    const int g = i / D, j = i % D;
    const size_t off = (static_cast<size_t>(bi) * prm.Hq + h0 + g) * D + j;
    float v;
    if (qdt == AXR_F32) {
      v = static_cast<const float*>(q)[off];
    } else if (qdt == AXR_F16) {
      v = __half2float(static_cast<const __half*>(q)[off]);
    } else {
      v = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(q)[off]) << 16);
    }
    if ((prm.sign[j >> 5] >> (j & 31)) & 1u) v = -v;
    qs[g][j] = v;
  }
  if (tid < 16) cent[tid] = prm.centroid[tid];
  __syncthreads();

  // 2. Walsh-Hadamard transform of each query, then 1/sqrt(d)
  for (int h = 1; h < D; h <<= 1) {
    for (int i = tid; i < GB * D / 2; i += kBlock) {
      const int g = i / (D / 2), k = i % (D / 2);
      const int lo = (k / h) * 2 * h + (k % h), hi = lo + h;
      const float a = qs[g][lo], b = qs[g][hi];
      qs[g][lo] = a + b;
      qs[g][hi] = a - b;
    }
    __syncthreads();
  }
  const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
  for (int i = tid; i < GB * D; i += kBlock) qs[i / D][i % D] *= inv_sqrt_d;
  __syncthreads();

  // 3. per-head fixed-point scale (fixed summation order: deterministic)
  const int wave = tid / 64, lane = tid % 64;
  const float cmax = fmaxf(fabsf(cent[0]), fabsf(cent[(1 << BITS) - 1]));
  for (int g = wave; g < GB; g += kBlock / 64) {
    float s = 0.0f;
    for (int j = lane; j < D; j += 64) s += fabsf(qs[g][j]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) {
      const float f = s * cmax * 1.0001f;
      int e = 0;
      if (f > 0.0f) frexpf(f, &e);           // f < 2^e
      int sh = 30 - e;
      sh = sh > 126 ? 126 : (sh < -126 ? -126 : sh);
      hscale[g] = ldexpf(1.0f, sh);
      hinv[g] = ldexpf(1.0f, -sh);
    }
  }
  __syncthreads();

  // 4. table of fixed-point group sums
  for (int e = tid; e < NG * NE * GB; e += kBlock) {
    const int g = e % GB;
    const int f = (e / GB) % NE;
    const int grp = e / (GB * NE);
    float v;
    if constexpr (P == 2) {
      v = fmaf(qs[g][2 * grp + 1], cent[f >> BITS], qs[g][2 * grp] * cent[f & ((1 << BITS) - 1)]);
    } else {
      v = qs[g][grp] * cent[f];
    }
    lut[e] = static_cast<int>(rintf(v * hscale[g]));
  }
  __syncthreads();

  float inv[GB];
#pragma unroll
  for (int g = 0; g < GB; ++g) inv[g] = hinv[g];

  // 5. stream the tile
  const int64_t t0 = static_cast<int64_t>(tile) * prm.tile_len;
  const int64_t t1 = (t0 + prm.tile_len < prm.T) ? t0 + prm.tile_len : prm.T;
  const size_t rowbase = static_cast<size_t>(row) * prm.t_cap;
  for (int64_t t = t0 + tid; t < t1; t += kBlock) {
    const uint4* rec = reinterpret_cast<const uint4*>(packed + (rowbase + t) * W);
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = rec[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
    const float nk = norms[rowbase + t];
    uint32_t acc[GB];
#pragma unroll
    for (int g = 0; g < GB; ++g) acc[g] = 0u;
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      const int pos = grp * FB, wi = pos >> 5, sh = pos & 31;
      uint32_t f;
      if (sh + FB <= 32) {
        f = (w[wi] >> sh) & FMASK;
      } else {
        f = ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & FMASK;
      }
      const int* ent = lut + (grp * NE + static_cast<int>(f)) * GB;
      if constexpr (GB % 4 == 0) {
#pragma unroll
        for (int g4 = 0; g4 < GB / 4; ++g4) {
          const int4 v = reinterpret_cast<const int4*>(ent)[g4];
          acc[4 * g4] += static_cast<uint32_t>(v.x);
          acc[4 * g4 + 1] += static_cast<uint32_t>(v.y);
          acc[4 * g4 + 2] += static_cast<uint32_t>(v.z);
          acc[4 * g4 + 3] += static_cast<uint32_t>(v.w);
        }
      } else if constexpr (GB == 2) {
        const int2 v = *reinterpret_cast<const int2*>(ent);
        acc[0] += static_cast<uint32_t>(v.x);
        acc[1] += static_cast<uint32_t>(v.y);
      } else {
        acc[0] += static_cast<uint32_t>(ent[0]);
      }
    }
#pragma unroll
    for (int g = 0; g < GB; ++g) {
      const float s = static_cast<float>(static_cast<int32_t>(acc[g])) * inv[g];
      scores[(static_cast<size_t>(bi) * prm.Hq + h0 + g) * prm.T + t] = nk * s;
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
template <int D, int BITS, int DT>
int launch_write_t(const void* keys, int64_t n, const WriteParams& p, uint32_t* packed,
                   float* norms, float* y, int mode, hipStream_t s) {
  constexpr int KPB = kBlock / (D / 32);
  const int64_t need = (n + KPB - 1) / KPB;
  const int grid = static_cast<int>(need < 4096 ? need : 4096);
  hipLaunchKernelGGL((write_kernel<D, BITS, DT>), dim3(grid), dim3(kBlock), 0, s, keys, n, p,
                     packed, norms, y, mode);
  return static_cast<int>(hipGetLastError());
}

template <int D, int BITS>
int launch_write_d(const void* keys, int dtype, int64_t n, const WriteParams& p,
                   uint32_t* packed, float* norms, float* y, int mode, hipStream_t s) {
  switch (dtype) {
    case AXR_F32: return launch_write_t<D, BITS, AXR_F32>(keys, n, p, packed, norms, y, mode, s);
    case AXR_F16: return launch_write_t<D, BITS, AXR_F16>(keys, n, p, packed, norms, y, mode, s);
    default: return launch_write_t<D, BITS, AXR_BF16>(keys, n, p, packed, norms, y, mode, s);
  }
}

template <int D>
int launch_write_b(const void* keys, int dtype, int64_t n, int b, const WriteParams& p,
                   uint32_t* packed, float* norms, float* y, int mode, hipStream_t s) {
  switch (b) {
    case 2: return launch_write_d<D, 2>(keys, dtype, n, p, packed, norms, y, mode, s);
    case 3: return launch_write_d<D, 3>(keys, dtype, n, p, packed, norms, y, mode, s);
    default: return launch_write_d<D, 4>(keys, dtype, n, p, packed, norms, y, mode, s);
  }
}

constexpr int kLutBudget = 64 * 1024;

constexpr int lut_bytes(int D, int BITS, int GB, int P) {
  return (D / P) * (1 << (P * BITS)) * GB * 4;
}

// Coordinates per table entry: pairs when the pair table fits the budget.
constexpr int pick_p(int D, int BITS, int GB) {
  return lut_bytes(D, BITS, GB, 2) <= kLutBudget ? 2 : 1;
}

template <int D, int BITS, int GB>
int launch_score_g(const void* q, int qdt, const uint32_t* packed, const float* norms, int B,
                   ScoreParams p, float* scores, hipStream_t s) {
  constexpr int P = pick_p(D, BITS, GB);
  constexpr int bytes = lut_bytes(D, BITS, GB, P);
  static_assert(bytes <= kLutBudget, "table exceeds the LDS budget");
  p.heads_per_block = GB;
  p.head_groups = p.G / GB;
  const int64_t rows = static_cast<int64_t>(B) * p.Hkv * p.head_groups;
  // aim for about 2048 blocks, tiles of at least 512 tokens
  int64_t tiles = (2048 + rows - 1) / rows;
  int64_t tile_len = (p.T + tiles - 1) / tiles;
  if (tile_len < 512) tile_len = 512;
  tile_len = (tile_len + kBlock - 1) / kBlock * kBlock;
  tiles = (p.T + tile_len - 1) / tile_len;
  p.tiles = static_cast<int>(tiles);
  p.tile_len = tile_len;
  const int64_t grid = rows * tiles;
  if (grid > 0x7FFFFFFF) return static_cast<int>(hipErrorInvalidValue);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&score_kernel<D, BITS, GB, P>),
      hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (attr != hipSuccess) return static_cast<int>(attr);
  hipLaunchKernelGGL((score_kernel<D, BITS, GB, P>), dim3(static_cast<unsigned>(grid)),
                     dim3(kBlock), bytes, s, q, qdt, packed, norms, scores, p);
  return static_cast<int>(hipGetLastError());
}

template <int D, int BITS, int GB>
constexpr bool table_fits() {
  return lut_bytes(D, BITS, GB, pick_p(D, BITS, GB)) <= kLutBudget;
}

// Largest heads-per-block in {8, 4, 2, 1} that divides G and whose table fits.
template <int D, int BITS>
int launch_score_b(const void* q, int qdt, const uint32_t* packed, const float* norms, int B,
                   const ScoreParams& p, float* scores, hipStream_t s) {
  if constexpr (table_fits<D, BITS, 8>()) {
    if (p.G % 8 == 0) return launch_score_g<D, BITS, 8>(q, qdt, packed, norms, B, p, scores, s);
  }
  if constexpr (table_fits<D, BITS, 4>()) {
    if (p.G % 4 == 0) return launch_score_g<D, BITS, 4>(q, qdt, packed, norms, B, p, scores, s);
  }
  if constexpr (table_fits<D, BITS, 2>()) {
    if (p.G % 2 == 0) return launch_score_g<D, BITS, 2>(q, qdt, packed, norms, B, p, scores, s);
  }
  return launch_score_g<D, BITS, 1>(q, qdt, packed, norms, B, p, scores, s);
}

template <int D>
int launch_score_d(const void* q, int qdt, const uint32_t* packed, const float* norms, int B,
                   int b, const ScoreParams& p, float* scores, hipStream_t s) {
  switch (b) {
    case 2: return launch_score_b<D, 2>(q, qdt, packed, norms, B, p, scores, s);
    case 3: return launch_score_b<D, 3>(q, qdt, packed, norms, B, p, scores, s);
    default: return launch_score_b<D, 4>(q, qdt, packed, norms, B, p, scores, s);
  }
}

}  // namespace

int launch_write(const void* keys, int dtype, int64_t n, int d, int b, const WriteParams& p,
                 uint32_t* packed, float* norms, float* y, int mode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 128: return launch_write_b<128>(keys, dtype, n, b, p, packed, norms, y, mode, s);
    case 256: return launch_write_b<256>(keys, dtype, n, b, p, packed, norms, y, mode, s);
    default: return launch_write_b<512>(keys, dtype, n, b, p, packed, norms, y, mode, s);
  }
}

int launch_score(const void* q, int q_dtype, const uint32_t* packed, const float* norms, int B,
                 int d, int b, const ScoreParams& p, float* scores, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 128: return launch_score_d<128>(q, q_dtype, packed, norms, B, b, p, scores, s);
    case 256: return launch_score_d<256>(q, q_dtype, packed, norms, B, b, p, scores, s);
    default: return launch_score_d<512>(q, q_dtype, packed, norms, B, b, p, scores, s);
  }
}

}  // namespace axr
