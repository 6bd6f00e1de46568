// Device helpers shared by the write and score kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace axr {

// Value held by lane (lane ^ M).  xor 1 / xor 2 are DPP quad permutations,
// xor 8 is DPP row_ror:8 inside a 16-lane row; xor 4 and xor 16 have no DPP
// control on this architecture and use ds_swizzle's bitmask mode (inside 32
// lanes); xor 32 crosses the half-waves through ds_bpermute.
template <int M>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  const int iv = static_cast<int>(v);
  if constexpr (M == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, false));
  } else if constexpr (M == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, false));
  } else if constexpr (M == 4 || M == 16) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(iv, (M << 10) | 0x1F));
  } else if constexpr (M == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, false));
  } else {
    static_assert(M == 32, "lane distance must be 1, 2, 4, 8, 16 or 32");
    return static_cast<uint32_t>(__shfl_xor(iv, 32));
  }
}

template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  return __uint_as_float(lane_xor_u32<M>(__float_as_uint(v)));
}

// Value held by lane (lane ^ 7) inside each group of 8 lanes: DPP
// row_half_mirror.
__device__ __forceinline__ float lane_mirror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}

// a * b rounded to fp32 on its own: never fused into a later add, so that
// the softmax partials and the row normalisation see the same scaled score
// (with a fused multiply-add in one place and a rounded product in the
// other, the row maximum's own exponent would differ from 0 by the product's
// rounding, which reaches whole units once |a * b| passes ~1e7).
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Right rotation of an N-word little-endian bit string by r bits, 0 <= r < 32.
template <int N>
__device__ __forceinline__ void rotate_right(uint32_t (&w)[N], uint32_t r) {
  uint32_t out[N];
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = __builtin_amdgcn_alignbit(w[(i + 1) % N], w[i], r);
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = out[i];
}

// Bits [pos, pos + width) of an N-word little-endian bit string; pos and
// width are compile-time after unrolling, width <= 32.
template <int N>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[N], int pos, int width) {
  const int wi = pos >> 5, sh = pos & 31;
  const uint32_t mask = width == 32 ? 0xFFFFFFFFu : ((1u << width) - 1u);
  if (sh + width <= 32) return (w[wi] >> sh) & mask;
  return __builtin_amdgcn_alignbit(w[(wi + 1) % N], w[wi], sh) & mask;
}

}  // namespace axr
