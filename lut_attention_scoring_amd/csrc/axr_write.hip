// Write-path kernels for gfx950: normalise, sign pattern, Walsh-Hadamard
// transform, Lloyd-Max bucketize and bit-pack each key of a KV cache.
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// an orthogonal transform on write makes every coordinate of a unit key
// close to N(0, 1/d), so a codebook fixed by (d, b) quantizes it; the
// indices are stored once and never dequantized.
//
// Layout: a key of d coordinates is held by LPK = d/32 adjacent lanes, lane u
// owning coordinates [32u, 32u + 32) in registers.  The transform is five
// butterfly stages inside each lane and log2(LPK) stages across lanes.  The
// 32 indices of a lane are exactly b words of the packed record, so every
// lane stores its own words and a wave writes one contiguous span.
//
// Lane stages are one fused multiply-add per coordinate, x + m * partner(x):
// inputs of lanes whose index has an odd number of set bits are negated on
// load (folded into the sign-pattern flip), which makes m = -1 for the lane
// with the stage bit clear and m = +1 for its partner and leaves every value
// un-negated after the last stage.
//
// Quantization compares z = H(s*k) (before the 1/(sqrt(d)||k||) scale)
// against thresholds multiplied by sqrt(d)||k||, by binary search on |z|
// over the positive thresholds of the symmetric codebook, then mirrors for
// z <= 0 (a coordinate equal to +0, and every coordinate of a zero key, takes
// the cell just below the middle threshold 0, as a value equal to a
// threshold does).  The b index bits of each coordinate are lane masks of
// compares; they are appended to the record words most significant bit
// first, one add-with-carry per bit.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "axr.h"
#include "axr_device.h"
#include "axr_internal.h"

namespace axr {
namespace {

constexpr int kBlock = 256;
typedef _Float16 half2_v __attribute__((ext_vector_type(2)));

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

// Block rotation of the comparison transform (IsoQuant, Abstract): the four
// coordinates v of a block, as the quaternion (w, x, y, z), become a v or,
// with a right factor, a v conj(c) (Hamilton products, 16 multiply-adds
// each).
template <bool kRight>
__device__ __forceinline__ void quat_block(float* v, const float (&a)[4], const float (&c)[4]) {
  const float vw = v[0], vx = v[1], vy = v[2], vz = v[3];
  const float tw = a[0] * vw - a[1] * vx - a[2] * vy - a[3] * vz;
  const float tx = a[0] * vx + a[1] * vw + a[2] * vz - a[3] * vy;
  const float ty = a[0] * vy - a[1] * vz + a[2] * vw + a[3] * vx;
  const float tz = a[0] * vz + a[1] * vy - a[2] * vx + a[3] * vw;
  if constexpr (kRight) {
    v[0] = tw * c[0] + tx * c[1] + ty * c[2] + tz * c[3];
    v[1] = -tw * c[1] + tx * c[0] - ty * c[3] + tz * c[2];
    v[2] = -tw * c[2] + tx * c[3] + ty * c[0] - tz * c[1];
    v[3] = -tw * c[3] - tx * c[2] + ty * c[1] + tz * c[0];
  } else {
    v[0] = tw;
    v[1] = tx;
    v[2] = ty;
    v[3] = tz;
  }
}

template <int DT>
struct Raw {
  static constexpr int kWords = DT == AXR_F32 ? 32 : 16;  // 32-bit words per lane chunk
};

// TF selects the transform: kWht (sign pattern + Walsh-Hadamard), or the
// block-quaternion comparison transforms kIsoFull / kIsoFast.
template <int D, int BITS, int DT, int TF>
__global__ __launch_bounds__(kBlock) void write_kernel(const void* __restrict__ keys, int64_t n,
                                                     WriteParams prm,
                                                     uint32_t* __restrict__ packed,
                                                     float* __restrict__ norms,
                                                     float* __restrict__ yout, int mode) {
  constexpr int LPK = D / 32;
  constexpr int KPB = kBlock / LPK;
  constexpr int W = D * BITS / 32;
  constexpr int NW = Raw<DT>::kWords;
  const int u = threadIdx.x % LPK;
  const int key_in_block = threadIdx.x / LPK;

  // Per-lane xor masks on the raw words: the sign pattern of this lane's 32
  // coordinates, plus a flip of everything when popcount(u) is odd.
  const uint32_t sw = prm.sign[u] ^ ((__popc(u) & 1) ? 0xFFFFFFFFu : 0u);
  uint32_t xm[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if constexpr (DT == AXR_F32) {
      xm[i] = ((sw >> i) & 1u) << 31;
    } else {
      xm[i] = (((sw >> (2 * i)) & 1u) << 15) | (((sw >> (2 * i + 1)) & 1u) << 31);
    }
  }
  const float m1 = (u & 1) ? 1.0f : -1.0f;
  const float m2 = (u & 2) ? 1.0f : -1.0f;
  const float m4 = (u & 4) ? 1.0f : -1.0f;
  const float m8 = (u & 8) ? 1.0f : -1.0f;
  float P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = prm.tpos[i];
  // quaternions of this lane's eight blocks (comparison transform only)
  float qa[8][4], qb[8][4];
  if constexpr (TF != kWht) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int m = 8 * u + k;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qa[k][c] = prm.quats[(m * 2) * 4 + c];
        qb[k][c] = TF == kIsoFull ? prm.quats[(m * 2 + 1) * 4 + c] : 0.0f;
      }
    }
  }

  for (int64_t base = static_cast<int64_t>(blockIdx.x) * KPB; base < n;
       base += static_cast<int64_t>(gridDim.x) * KPB) {
    const int64_t key = base + key_in_block;
    const bool valid = key < n;
    const int64_t kc = valid ? key : n - 1;
    const size_t off = static_cast<size_t>(kc) * D + static_cast<size_t>(u) * 32;

    uint32_t raw[NW];
    {
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const char*>(keys) + off * (DT == AXR_F32 ? 4 : 2));
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const uint4 v = src[i];
        raw[4 * i] = v.x;
        raw[4 * i + 1] = v.y;
        raw[4 * i + 2] = v.z;
        raw[4 * i + 3] = v.w;
      }
    }

    // sum of squares (sign-independent), first butterfly stage fused with
    // the conversion to fp32
    float ss = 0.0f;
    float x[32];
    if constexpr (TF != kWht) {
      // comparison transform: plain conversion, then the block rotations
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float lo, hi;
        if constexpr (DT == AXR_F16) {
          const half2_v h2 = __builtin_bit_cast(half2_v, raw[i]);
          ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
          lo = static_cast<float>(h2.x);
          hi = static_cast<float>(h2.y);
        } else if constexpr (DT == AXR_BF16) {
          lo = __uint_as_float(raw[i] << 16);
          hi = __uint_as_float(raw[i] & 0xFFFF0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        } else {
          lo = __uint_as_float(raw[2 * i]);
          hi = __uint_as_float(raw[2 * i + 1]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
        x[2 * i] = lo;
        x[2 * i + 1] = hi;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) quat_block<TF == kIsoFull>(&x[4 * k], qa[k], qb[k]);
    } else if constexpr (DT == AXR_F16) {
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
        const uint32_t f = raw[i] ^ xm[i];
        const float lo = __uint_as_float(f << 16);
        const float hi = __uint_as_float(f & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
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
    if constexpr (LPK >= 2) ss += lane_xor<1>(ss);
    if constexpr (LPK >= 4) ss += lane_xor<2>(ss);
    if constexpr (LPK >= 8) ss += lane_xor<4>(ss);
    if constexpr (LPK >= 16) ss += lane_xor<8>(ss);
    const float nrm = sqrtf(ss);

    if constexpr (TF == kWht) {
      reg_stage<2>(x);
      reg_stage<4>(x);
      reg_stage<8>(x);
      reg_stage<16>(x);
      if constexpr (LPK >= 2) lane_stage<1>(x, m1);
      if constexpr (LPK >= 4) lane_stage<2>(x, m2);
      if constexpr (LPK >= 8) lane_stage<4>(x, m4);
      if constexpr (LPK >= 16) lane_stage<8>(x, m8);
    }

    if (mode == kWriteQuantize) {
      float S[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) S[i] = P[i] * nrm;
      // Record words filled most significant bit first: walking the bit
      // positions downwards, each index bit is appended to its word as
      // w + w + bit (one add with carry-in).
      uint32_t words[BITS];
#pragma unroll
      for (int i = 0; i < BITS; ++i) words[i] = 0u;
#pragma unroll
      for (int r = 31; r >= 0; --r) {
        uint64_t bit[BITS];                     // lane masks
        index_bits<BITS>(x[r], S, bit);
#pragma unroll
        for (int k = BITS - 1; k >= 0; --k) {
          const int wi = (r * BITS + k) >> 5;
          words[wi] = append_bit(words[wi], bit[k]);
        }
      }
      // destination row: the key's own index, or its cache slot when appending
      int64_t row = key;
      bool store = valid;
      if (prm.pos != nullptr && valid) {
        const int32_t slot = prm.pos[static_cast<uint32_t>(key) / static_cast<uint32_t>(prm.Hkv)];
        store = slot >= 0 && slot < prm.t_cap;
        row = key * prm.t_cap + slot;
      }
      if (store) {
        uint32_t* dst = packed + static_cast<size_t>(row) * W + u * BITS;
        if constexpr (BITS == 2) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else if constexpr (BITS == 4) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        } else {
#pragma unroll
          for (int i = 0; i < BITS; ++i) dst[i] = words[i];
        }
        if (u == 0) norms[row] = nrm;
      }
    } else {
      float scale = prm.inv_sqrt_d;
      if (mode == kWriteTransformNormalized) scale = nrm > 0.0f ? prm.inv_sqrt_d / nrm : 0.0f;
      if (valid) {
        float4* dst = reinterpret_cast<float4*>(yout + static_cast<size_t>(key) * D +
                                                static_cast<size_t>(u) * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          dst[i] = make_float4(x[4 * i] * scale, x[4 * i + 1] * scale, x[4 * i + 2] * scale,
                               x[4 * i + 3] * scale);
      }
    }
  }
}

template <int D, int BITS, int DT, int TF>
int launch_t(const void* keys, int64_t n, const WriteParams& p, uint32_t* packed, float* norms,
             float* y, int mode, hipStream_t s) {
  constexpr int KPB = kBlock / (D / 32);
  const int64_t need = (n + KPB - 1) / KPB;
  const int grid = static_cast<int>(need < 4096 ? need : 4096);
  hipLaunchKernelGGL((write_kernel<D, BITS, DT, TF>), dim3(grid), dim3(kBlock), 0, s, keys, n,
                     p, packed, norms, y, mode);
  return static_cast<int>(hipGetLastError());
}

template <int D, int BITS, int DT>
int launch_tf(const void* keys, int64_t n, const WriteParams& p, uint32_t* packed,
              float* norms, float* y, int mode, int tf, hipStream_t s) {
  switch (tf) {
    case kIsoFull: return launch_t<D, BITS, DT, kIsoFull>(keys, n, p, packed, norms, y, mode, s);
    case kIsoFast: return launch_t<D, BITS, DT, kIsoFast>(keys, n, p, packed, norms, y, mode, s);
    default: return launch_t<D, BITS, DT, kWht>(keys, n, p, packed, norms, y, mode, s);
  }
}

template <int D, int BITS>
int launch_dt(const void* keys, int dtype, int64_t n, const WriteParams& p, uint32_t* packed,
              float* norms, float* y, int mode, int tf, hipStream_t s) {
  switch (dtype) {
    case AXR_F32: return launch_tf<D, BITS, AXR_F32>(keys, n, p, packed, norms, y, mode, tf, s);
    case AXR_F16: return launch_tf<D, BITS, AXR_F16>(keys, n, p, packed, norms, y, mode, tf, s);
    default: return launch_tf<D, BITS, AXR_BF16>(keys, n, p, packed, norms, y, mode, tf, s);
  }
}

template <int D>
int launch_b(const void* keys, int dtype, int64_t n, int b, const WriteParams& p,
             uint32_t* packed, float* norms, float* y, int mode, int tf, hipStream_t s) {
  switch (b) {
    case 2: return launch_dt<D, 2>(keys, dtype, n, p, packed, norms, y, mode, tf, s);
    case 3: return launch_dt<D, 3>(keys, dtype, n, p, packed, norms, y, mode, tf, s);
    default: return launch_dt<D, 4>(keys, dtype, n, p, packed, norms, y, mode, tf, s);
  }
}

}  // namespace

int launch_write(const void* keys, int dtype, int64_t n, int d, int b, const WriteParams& p,
                 uint32_t* packed, float* norms, float* y, int mode, void* stream, int tf) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 128: return launch_b<128>(keys, dtype, n, b, p, packed, norms, y, mode, tf, s);
    case 256: return launch_b<256>(keys, dtype, n, b, p, packed, norms, y, mode, tf, s);
    default: return launch_b<512>(keys, dtype, n, b, p, packed, norms, y, mode, tf, s);
  }
}

}  // namespace axr
