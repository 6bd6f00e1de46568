// Per-lane write-path arithmetic shared by the kernels that quantize keys:
// the write kernel, and the score kernel when it quantizes the keys it
// scores (quantize-and-score).  A key of d coordinates is held by LPK = d/32 adjacent lanes
// of a wave (lane u owns the 32 coordinates of block lane_block(u), see
// below); every lane of the wave must be active, since the transform
// exchanges values across lanes.
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

// The block of 32 coordinates that lane u of a key holds.  The lane stages
// of the transform pair lanes u and u ^ M for the masks M = 1, 2, 7, 8 (the
// ones DPP reaches: quad permutations, the mirror inside 8 lanes, and a
// rotation by 8 inside 16; lane xor 4 has no DPP pattern).  Over the basis
// 1, 2, 7, 8 of the lane index, these stages are the butterflies of the
// 16-point Hadamard transform on the basis coordinates, which are the bits
// of b(u) = u ^ (3 if bit 2 of u is set): b is linear and maps the masks to
// 1, 2, 4, 8.  So lane u loads block b(u), its multipliers and sign-pattern
// bits follow the bits of b(u), and it ends with block b(u) of the output.
// With at most 4 lanes per key only masks 1 and 2 occur and b(u) = u.
template <int LPK>
__device__ __forceinline__ int lane_block(int u) {
  return LPK >= 8 ? (u ^ ((u & 4) ? 3 : 0)) : u;
}

// One butterfly stage across lanes with lane mask M (7 standing for the
// mirror inside 8 lanes, see lane_block): x <- x + m * x[lane ^ M].  Each is
// a single v_fmac_f32 with a DPP source operand; each block of 16 starts
// with s_nop 1 because a DPP read of a VGPR needs two wait states after the
// VALU write of that VGPR, and the instructions of a block read and write
// disjoint registers.
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
#pragma unroll
  for (int o = 0; o < 32; o += 16) {
    if constexpr (M == 1) {
      AXR_FMAC16("quad_perm:[1,0,3,2]");
    } else if constexpr (M == 2) {
      AXR_FMAC16("quad_perm:[2,3,0,1]");
    } else if constexpr (M == 7) {
      AXR_FMAC16("row_half_mirror");
    } else {
      static_assert(M == 8, "lane mask must be 1, 2, 7 or 8");
      AXR_FMAC16("row_ror:8");
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

// a + b + (this lane's bit of m), one add whose carry-in is the lane mask.
__device__ __forceinline__ uint32_t add_with_carry(uint32_t a, uint32_t b, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %3, %4" : "=v"(r), "=s"(carry_out) : "v"(a), "v"(b), "s"(m));
  return r;
}

// 32-bit words of one lane's 32 raw coordinates.
template <int DT>
struct RawWords {
  static constexpr int kWords = DT == AXR_F32 ? 32 : 16;
};

// ||k||: the sum of squares of a lane's coordinates added over the key's
// lanes (partners at lane masks 1, 2, 7, 8, which span every lane of the key).
template <int LPK>
__device__ __forceinline__ float key_norm(float ss) {
  if constexpr (LPK >= 2) ss += lane_xor<1>(ss);
  if constexpr (LPK >= 4) ss += lane_xor<2>(ss);
  if constexpr (LPK >= 8) ss += lane_mirror8(ss);
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

// First butterfly stage of raw words o .. o + 3 (fp16 or bf16 pairs): x[2i]
// and x[2i + 1] are the dot products of raw[i] with sg[i] and with sg[i]
// negated in its high half.  A VALU read or write of a dot product's result
// needs three wait states after it on this architecture, which the compiler
// does not insert for inline asm: the trailing s_nop 2 provides them.
#define AXR_DOT2X8(OP)                                                              \
  asm(OP " %0, %8, %12, 0\n\t" OP " %1, %8, %12, 0 neg_hi:[0,1,0]\n\t"                \
      OP " %2, %9, %13, 0\n\t" OP " %3, %9, %13, 0 neg_hi:[0,1,0]\n\t"                \
      OP " %4, %10, %14, 0\n\t" OP " %5, %10, %14, 0 neg_hi:[0,1,0]\n\t"              \
      OP " %6, %11, %15, 0\n\t" OP " %7, %11, %15, 0 neg_hi:[0,1,0]\n\t"              \
      "s_nop 2"                                                                     \
      : "=&v"(x[2 * o]), "=&v"(x[2 * o + 1]), "=&v"(x[2 * o + 2]), "=&v"(x[2 * o + 3]), \
        "=&v"(x[2 * o + 4]), "=&v"(x[2 * o + 5]), "=&v"(x[2 * o + 6]), "=&v"(x[2 * o + 7]) \
      : "v"(raw[o]), "v"(raw[o + 1]), "v"(raw[o + 2]), "v"(raw[o + 3]), "v"(sg[o]),    \
        "v"(sg[o + 1]), "v"(sg[o + 2]), "v"(sg[o + 3]))

// The sign pattern and the Walsh-Hadamard transform for one lane of a key,
// the lane holding coordinate block blk = lane_block(u).  transform() leaves
// z = H (s * k) (no 1/sqrt(d)) in x and returns ||k||.  The per-word sign
// masks depend only on the block: kernels keep them in LDS (fill_sign_masks,
// one row of NW words per block, read back with 16-byte broadcast loads by
// transform_lds) rather than in NW registers per lane.
template <int D, int DT>
struct WhtLane {
  static constexpr int LPK = D / 32;
  static constexpr int NW = RawWords<DT>::kWords;
  static constexpr bool kDotStage = DT != AXR_F32 && LPK >= 8;
  float m1, m2, m7, m8;

  // Word i of the block's sign masks, from its sign word sw (the sign
  // pattern of the block's 32 coordinates, times -1 throughout when
  // popcount(blk) is odd, which makes every lane stage a single fused
  // multiply-add): for fp16 / bf16 the pair (+-1, +-1) in the key's format
  // that multiplies the word's two coordinates (only its sign bits without
  // the dot product stage); for fp32 the sign bit to xor into coordinate i.
  static __device__ __forceinline__ uint32_t sign_mask(uint32_t sw, int i) {
    constexpr uint32_t one = DT == AXR_F16 ? 0x3C00u : 0x3F80u;   // 1.0 in the half format
    if constexpr (DT == AXR_F32) {
      return ((sw >> i) & 1u) << 31;
    } else {
      return ((((sw >> (2 * i)) & 1u) << 15) | (((sw >> (2 * i + 1)) & 1u) << 31)) |
             (kDotStage ? one * 0x10001u : 0u);
    }
  }

  static __device__ __forceinline__ uint32_t sign_word(const uint32_t* sign_words, int blk) {
    return sign_words[blk] ^ ((__popc(blk) & 1) ? 0xFFFFFFFFu : 0u);
  }

  // All LPK rows of sign masks into lds[LPK * NW] (block b's row at b * NW),
  // by the calling block's threads; the caller synchronises before use.
  static __device__ __forceinline__ void fill_sign_masks(uint32_t* lds, const uint32_t* sign_words,
                                                         int tid, int nthreads) {
    for (int t = tid; t < LPK * NW; t += nthreads) lds[t] = sign_mask(sign_word(sign_words, t / NW), t % NW);
  }

  // The lane-stage multipliers from the bits of blk.
  __device__ __forceinline__ void init(int blk) {
    m1 = (blk & 1) ? 1.0f : -1.0f;
    m2 = (blk & 2) ? 1.0f : -1.0f;
    m7 = (blk & 4) ? 1.0f : -1.0f;
    m8 = (blk & 8) ? 1.0f : -1.0f;
  }

  // The transform with the block's sign masks read from its LDS row
  // (16-byte aligned).
  __device__ __forceinline__ float transform_lds(const uint32_t (&raw)[NW], float (&x)[32],
                                                 const uint4* row) const {
    uint32_t sg[NW];
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = row[i];
      sg[4 * i] = v.x;
      sg[4 * i + 1] = v.y;
      sg[4 * i + 2] = v.z;
      sg[4 * i + 3] = v.w;
    }
    return transform(raw, x, sg);
  }

  __device__ __forceinline__ float transform(const uint32_t (&raw)[NW], float (&x)[32],
                                             const uint32_t (&sg)[NW]) const {
    // Sum of squares (sign-independent), and the first butterfly stage
    // fused with the sign pattern and the conversion to fp32.  For the
    // half formats with d >= 256 that stage is a dot product of the raw
    // word with its signs, (lo, hi) . (s0, s1) and (lo, hi) . (s0, -s1) (the
    // second through the instruction's negate-high modifier): two
    // instructions per word instead of four.  The products are exact; the
    // hardware's sum is within 1 ulp of the larger term (not always the
    // nearest fp32 value; exact when a term is zero), and a sum of two zeros
    // may come out as +0 where fp32 addition gives -0, which takes the same
    // index.  At d = 128 the sign flip, conversion and add / subtract
    // measured faster (the dot products' wait states sit on a shorter loop).
    float ss = 0.0f;
    if constexpr (DT == AXR_F16 || DT == AXR_BF16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (DT == AXR_F16) {
          const half2_v h2 = __builtin_bit_cast(half2_v, raw[i]);
          ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
        } else {
          const bf16x2_v b2 = __builtin_bit_cast(bf16x2_v, raw[i]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(b2, b2, ss, false);
        }
      }
      if constexpr (kDotStage) {
#pragma unroll
        for (int o = 0; o < 16; o += 4) {
          if constexpr (DT == AXR_F16) {
            AXR_DOT2X8("v_dot2_f32_f16");
          } else {
            AXR_DOT2X8("v_dot2_f32_bf16");
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t f = raw[i] ^ sg[i];
          if constexpr (DT == AXR_F16) {
            // lo + hi, lo - hi straight from the two fp16 halves
            asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
                : "=v"(x[2 * i]) : "v"(f));
            asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
                : "=v"(x[2 * i + 1]) : "v"(f));
          } else {
            const float lo = __uint_as_float(f << 16);
            const float hi = __uint_as_float(f & 0xFFFF0000u);
            x[2 * i] = lo + hi;
            x[2 * i + 1] = lo - hi;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float lo = __uint_as_float(raw[2 * i] ^ sg[2 * i]);
        const float hi = __uint_as_float(raw[2 * i + 1] ^ sg[2 * i + 1]);
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
    if constexpr (LPK >= 8) lane_stage<7>(x, m7);
    if constexpr (LPK >= 16) lane_stage<8>(x, m8);
    return nrm;
  }
};
#undef AXR_DOT2X8

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
// time, highest coordinate first, each appended in one add with carry-in:
// (w << 4) + cnt + (u > un).  (At b = 3 the threshold search measured as
// fast: three compares and a select against six VALU slots here.)
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
    words[r >> 3] = add_with_carry(words[r >> 3] << 4, e.x,
                                   __builtin_amdgcn_ballot_w64(u > __uint_as_float(e.y)));
  }
}

}  // namespace axr
