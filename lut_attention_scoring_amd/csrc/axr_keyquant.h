// Per-lane write-path arithmetic shared by the kernels that quantize keys:
// the write kernel, and the score kernel when it appends the new key of a
// decode step.  A key of d coordinates is held by LPK = d/32 adjacent lanes
// of a wave (lane u owns coordinates [32u, 32u + 32)); every lane of the
// wave must be active, since the transform exchanges values across lanes.
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// the seeded sign pattern and normalised Walsh-Hadamard transform make each
// coordinate of a unit key close to N(0, 1/d); the Lloyd-Max codebook of
// that density turns it into a b-bit index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "axr.h"
#include "axr_device.h"

namespace axr {

typedef _Float16 half2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// One butterfly stage across lanes at distance M (see the file comment):
// x <- x + m * x[lane ^ M].  Distances 1, 2 and 8 are single v_fmac_f32 with a
// DPP source operand; each block of 16 starts with s_nop 1 because a DPP read
// of a VGPR needs two wait states after the VALU write of that VGPR, and the
// instructions of a block read and write disjoint registers.  Distance 4 has
// no DPP pattern and goes through ds_swizzle.
#define AXR_FMAC16(CTRL)                                                              \
  asm("s_nop 1\n\t"                                                                  \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"           \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"         \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"         \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"         \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"         \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"         \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf"               \
      : "+v"(x[o + 0]), "+v"(x[o + 1]), "+v"(x[o + 2]), "+v"(x[o + 3]), "+v"(x[o + 4]),  \
        "+v"(x[o + 5]), "+v"(x[o + 6]), "+v"(x[o + 7]), "+v"(x[o + 8]), "+v"(x[o + 9]),  \
        "+v"(x[o + 10]), "+v"(x[o + 11]), "+v"(x[o + 12]), "+v"(x[o + 13]),             \
        "+v"(x[o + 14]), "+v"(x[o + 15])                                                \
      : "v"(m))

template <int M>
__device__ __forceinline__ void lane_stage(float (&x)[32], float m) {
  if constexpr (M == 4) {
#pragma unroll
    for (int r = 0; r < 32; ++r) x[r] = fmaf(lane_xor<4>(x[r]), m, x[r]);
  } else {
#pragma unroll
    for (int o = 0; o < 32; o += 16) {
      if constexpr (M == 1) {
        AXR_FMAC16("quad_perm:[1,0,3,2]");
      } else if constexpr (M == 2) {
        AXR_FMAC16("quad_perm:[2,3,0,1]");
      } else {
        static_assert(M == 8, "lane distance must be 1, 2, 4 or 8");
        AXR_FMAC16("row_ror:8");
      }
    }
  }
}
#undef AXR_FMAC16

// Butterfly stages with half-distance H (1, 2, ..., 16) inside a lane.
template <int H>
__device__ __forceinline__ void reg_stage(float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if ((i & H) == 0) {
      const float a = x[i], b = x[i + H];
      x[i] = a + b;
      x[i + H] = a - b;
    }
  }
}

// Bits of one coordinate's index, most significant first.  With
// p = (z > 0) and a binary search on |z| against the positive thresholds
// (decisions c_k, most significant first), the positive side has index
// HALF + cell = (1, c_{b-2}, ..., c_0) and the mirrored negative side
// HALF - 1 - cell = (0, !c_{b-2}, ..., !c_0): every lower bit is c_k == p.
// z = +0 and z = -0 take the cell just below the middle threshold (0), as
// the count of thresholds strictly below z requires, so a zero key needs no
// special case.
template <int BITS>
__device__ __forceinline__ void index_bits(float z, const float (&S)[8], uint64_t (&bit)[BITS]) {
  const uint64_t p = __builtin_amdgcn_ballot_w64(z > 0.0f);
  const float a = fabsf(z);
  bit[BITS - 1] = p;
  if constexpr (BITS == 2) {
    bit[0] = ~(__builtin_amdgcn_ballot_w64(a > S[0]) ^ p);
  } else if constexpr (BITS == 3) {
    const bool c1 = a > S[1];
    const bool c0 = a > (c1 ? S[2] : S[0]);
    bit[1] = ~(__builtin_amdgcn_ballot_w64(c1) ^ p);
    bit[0] = ~(__builtin_amdgcn_ballot_w64(c0) ^ p);
  } else {
    static_assert(BITS == 4, "b must be 2, 3 or 4");
    const bool c2 = a > S[3];
    const bool c1 = a > (c2 ? S[5] : S[1]);
    const bool c0 = a > (c2 ? (c1 ? S[6] : S[4]) : (c1 ? S[2] : S[0]));
    bit[2] = ~(__builtin_amdgcn_ballot_w64(c2) ^ p);
    bit[1] = ~(__builtin_amdgcn_ballot_w64(c1) ^ p);
    bit[0] = ~(__builtin_amdgcn_ballot_w64(c0) ^ p);
  }
}

// w + w + (this lane's bit of m): appends one bit below w's bits, as one add
// whose carry-in is the lane mask (the compiler would turn the shift-add
// into shifts, selects and ors).
__device__ __forceinline__ uint32_t append_bit(uint32_t w, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
  return r;
}

// 32-bit words of one lane's 32 raw coordinates.
template <int DT>
struct RawWords {
  static constexpr int kWords = DT == AXR_F32 ? 32 : 16;
};

// ||k||: the sum of squares of a lane's coordinates added over the key's lanes.
template <int LPK>
__device__ __forceinline__ float key_norm(float ss) {
  if constexpr (LPK >= 2) ss += lane_xor<1>(ss);
  if constexpr (LPK >= 4) ss += lane_xor<2>(ss);
  if constexpr (LPK >= 8) ss += lane_xor<4>(ss);
  if constexpr (LPK >= 16) ss += lane_xor<8>(ss);
  return sqrtf(ss);
}

// A key whose squares underflow fp32 (every |k_j| below ~1e-19) comes out of
// key_norm far below 2^-50, and one whose squares overflow (|k_j| above
// ~1.8e19) as inf.  Such a norm is taken again from the key's transformed
// coordinates x scaled by 2^64 or 2^-64 (exact): the transform keeps the
// norm up to the factor 1 / inv_sqrt_d.  All lanes of a key take the same
// branch, so the lane exchanges stay among active lanes.
template <int LPK>
__device__ __forceinline__ float rescued_key_norm(float nrm, const float (&x)[32],
                                                  float inv_sqrt_d) {
  if (nrm >= 0x1p-50f && nrm <= 0x1p50f) return nrm;
  const bool tiny = !(nrm >= 0x1p-50f);         // also NaN, which stays NaN
  const float up = tiny ? 0x1p64f : 0x1p-64f;
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float t = x[i] * up;
    ss = fmaf(t, t, ss);
  }
  return (key_norm<LPK>(ss) * (tiny ? 0x1p-64f : 0x1p64f)) * inv_sqrt_d;
}

// The sign pattern and the Walsh-Hadamard transform for lane u of a key.
// transform() leaves z = H (s * k) (no 1/sqrt(d)) in x and returns ||k||.
template <int D, int DT>
struct WhtLane {
  static constexpr int LPK = D / 32;
  static constexpr int NW = RawWords<DT>::kWords;
  uint32_t xm[NW];
  float m1, m2, m4, m8;

  // Per-lane xor masks on the raw words: the sign pattern of this lane's 32
  // coordinates, plus a flip of everything when popcount(u) is odd (which
  // makes every lane stage a single fused multiply-add).
  __device__ __forceinline__ void init(const uint32_t* sign_words, int u) {
    const uint32_t sw = sign_words[u] ^ ((__popc(u) & 1) ? 0xFFFFFFFFu : 0u);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      if constexpr (DT == AXR_F32) {
        xm[i] = ((sw >> i) & 1u) << 31;
      } else {
        xm[i] = (((sw >> (2 * i)) & 1u) << 15) | (((sw >> (2 * i + 1)) & 1u) << 31);
      }
    }
    m1 = (u & 1) ? 1.0f : -1.0f;
    m2 = (u & 2) ? 1.0f : -1.0f;
    m4 = (u & 4) ? 1.0f : -1.0f;
    m8 = (u & 8) ? 1.0f : -1.0f;
  }

  __device__ __forceinline__ float transform(const uint32_t (&raw)[NW], float (&x)[32]) const {
    // sum of squares (sign-independent), first butterfly stage fused with
    // the conversion to fp32
    float ss = 0.0f;
    if constexpr (DT == AXR_F16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t r = raw[i];
        const half2_v h2 = __builtin_bit_cast(half2_v, r);
        ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
        const uint32_t f = r ^ xm[i];
        // first butterfly straight from the two fp16 halves: lo + hi, lo - hi
        asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
            : "=v"(x[2 * i]) : "v"(f));
        asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
            : "=v"(x[2 * i + 1]) : "v"(f));
      }
    } else if constexpr (DT == AXR_BF16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16x2_v b2 = __builtin_bit_cast(bf16x2_v, raw[i]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ss, false);
        const uint32_t f = raw[i] ^ xm[i];
        const float lo = __uint_as_float(f << 16);
        const float hi = __uint_as_float(f & 0xFFFF0000u);
        x[2 * i] = lo + hi;
        x[2 * i + 1] = lo - hi;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float lo = __uint_as_float(raw[2 * i] ^ xm[2 * i]);
        const float hi = __uint_as_float(raw[2 * i + 1] ^ xm[2 * i + 1]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
        x[2 * i] = lo + hi;
        x[2 * i + 1] = lo - hi;
      }
    }
    const float nrm = key_norm<LPK>(ss);
    reg_stage<2>(x);
    reg_stage<4>(x);
    reg_stage<8>(x);
    reg_stage<16>(x);
    if constexpr (LPK >= 2) lane_stage<1>(x, m1);
    if constexpr (LPK >= 4) lane_stage<2>(x, m2);
    if constexpr (LPK >= 8) lane_stage<4>(x, m4);
    if constexpr (LPK >= 16) lane_stage<8>(x, m8);
    return nrm;
  }
};

// The b record words of a lane's 32 coordinates x against the positive
// thresholds S (already multiplied by the key's scale), filled most
// significant bit first: walking the bit positions downwards, each index bit
// is appended to its word as w + w + bit (one add with carry-in).
template <int BITS>
__device__ __forceinline__ void quantize_lane(const float (&x)[32], const float (&S)[8],
                                              uint32_t (&words)[BITS]) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) words[i] = 0u;
#pragma unroll
  for (int r = 31; r >= 0; --r) {
    uint64_t bit[BITS];                         // lane masks
    index_bits<BITS>(x[r], S, bit);
#pragma unroll
    for (int k = BITS - 1; k >= 0; --k) {
      const int wi = (r * BITS + k) >> 5;
      words[wi] = append_bit(words[wi], bit[k]);
    }
  }
}

// The 4-bit index of each of a lane's 32 coordinates from the cell table:
// u = z kc + kCellMid (kc = K / ||k||, K the table's scale) falls in cell c,
// which holds cnt thresholds below it and at most one more inside it, at
// position un = t K + kCellMid on the same scale; the index is
// cnt + (u > un), the number of thresholds strictly below z (z > t ||k||
// taken on the cell scale, where the rounding of u and un is ~2^-17 of a
// cell, a few 1e-7 of a threshold gap).  The host keeps |u - kCellMid| two
// cells short of the table's ends for every key whose norm lies in the
// table's range (the only keys that get here), and a non-finite u converts
// to 0, so c needs no clamp.  Indices fill the record words a nibble at a
// time, highest coordinate first.
__device__ __forceinline__ void quantize_cells(const float (&x)[32], float kc,
                                               const uint2* cells, uint32_t (&words)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) words[i] = 0u;
#pragma unroll
  for (int r = 31; r >= 0; --r) {
    const float u = fmaf(x[r], kc, kCellMid);
    uint32_t c;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(c) : "v"(u));   // saturating: < 0 -> 0
    const uint2 e = cells[c];
    const uint32_t idx = e.x + (u > __uint_as_float(e.y) ? 1u : 0u);
    words[r >> 3] = (words[r >> 3] << 4) | idx;
  }
}

}  // namespace axr
