// Read-path kernel for gfx950: attention scores straight from packed
// quantization indices, by table lookup, with no inverse transform.
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// the query is turned once into a table of products q'_j * c_k and each key's
// score is its stored norm times the sum of the table entries its indices
// select.
//
// Design (one block = up to 8 query heads of one (batch, KV head) row, one
// tile of tokens):
//   * prologue: q' = H (s * q) / sqrt(d) for the block's heads (LDS), a
//     power-of-two fixed-point scale per head, and a table of group sums in
//     LDS.  A group is P = 2 adjacent coordinates (a 2b-bit field of the
//     packed record, so no index reshuffling), P = 4 for 2-bit indices at
//     d = 128 (8-bit fields), or P = 1 when the pair table would not fit.
//     One table entry is 16 bytes: the group sum for 4 heads.  Entries are int32: each coordinate term q'_j c_k rounded to a
//     unit of the head's scale, which puts sum_j |q'_j| max_k |c_k| in
//     [2^30, 2^31) units, and integer accumulation is exact, so the score's
//     only roundings are those terms and the final fp32 multiply.  The
//     signed half table of 4-bit pairs at d = 128 (see ScoreShape) keeps
//     fp32 entries instead, each the sum of its two rounded terms, summed in
//     fp32.
//   * loop: a key is read by LPK = d/32 adjacent lanes, lane u owning the
//     32 coordinates [32u, 32u+32) = b words of the record, so a wave reads
//     a contiguous span of records.  Each lane looks up its groups (several
//     lookups issued before any of their sums), the lanes of a key sum their
//     partial results across lanes, and each lane writes the scores of its
//     heads.
//   * work split: one block per CU; the block's tile is cut into units of
//     one wave's keys, handed out by a per-block LDS counter, so the waves
//     that the SIMD's issue arbitration favours take more units and all
//     waves of the block finish together.  The blocks of a row's head
//     groups, which read the same records, run on one XCD.
//   * quantize-and-score (mode kFused, d = 128, b = 2 or 3, one head group of
//     up to four heads, or eight at b = 3 with two tables):
//     each wave loads the raw keys of its unit instead of records, quantizes
//     them with the write path's lane arithmetic (lane u holds block u,
//     whose b record words it then looks up), stores records and norms, and
//     scores them from registers, so the records are never read back.
//   * LDS banks: 16-byte reads are conflict-free when the 16 lanes of a
//     quarter-wave touch 16 different 16-byte columns of a 256-byte row.  The
//     table puts group v of lane-chunk u in column (v + KPG*u) mod 16 and each
//     lane walks its groups starting at an offset k (its key's slot in the
//     quarter-wave), after rotating its record by k fields, so the 16 lanes
//     always hit 16 distinct columns whatever the indices are.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <type_traits>

#include "axr.h"
#include "axr_device.h"
#include "axr_internal.h"
#include "axr_keyquant.h"

namespace axr {
namespace {

// k + s[lane ^ M] as one v_add_u32 with a DPP source (M = 1 or 2, quad
// permutations).  The leading s_nop 1 gives the two wait states a DPP read
// needs after the VALU write of its source.
template <int M>
__device__ __forceinline__ uint32_t dpp_add(uint32_t k, uint32_t s) {
  if constexpr (M == 1) {
    asm("s_nop 1\n\tv_add_u32_dpp %0, %1, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(k) : "v"(s));
  } else {
    static_assert(M == 2, "quad distances only");
    asm("s_nop 1\n\tv_add_u32_dpp %0, %1, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(k) : "v"(s));
  }
  return k;
}

// Sum over the 4 lanes of a quad, scattered: a[i] of lane u holds head
// (u ^ i), so lane u ends with the total of head u.  Each step keeps the half
// whose heads match the lane's own bit and sends the other half, which in the
// partner's numbering is exactly the half it keeps: no selects are needed.
__device__ __forceinline__ uint32_t quad_reduce_scatter(const uint32_t (&a)[4]) {
  const uint32_t k0 = dpp_add<2>(a[0], a[2]);   // heads u and u^1 (+ partner u^2)
  const uint32_t k1 = dpp_add<2>(a[1], a[3]);
  return dpp_add<1>(k0, k1);                    // head u
}

// The same for fp32 partial sums (v_add_f32 with a DPP source).
template <int M>
__device__ __forceinline__ float dpp_addf(float k, float s) {
  if constexpr (M == 1) {
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "+v"(k) : "v"(s));
  } else {
    static_assert(M == 2, "quad distances only");
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "+v"(k) : "v"(s));
  }
  return k;
}

__device__ __forceinline__ float quad_reduce_scatter(const float (&a)[4]) {
  const float k0 = dpp_addf<2>(a[0], a[2]);
  const float k1 = dpp_addf<2>(a[1], a[3]);
  return dpp_addf<1>(k0, k1);
}

// Running (max, sum of exp(x - max)) of a stream of finite values x, one
// exponential per value; starts from (-inf, 0).
__device__ __forceinline__ void lse_push(float& m, float& l, float x) {
  const float dx = x - m;                       // +inf while the stream is empty
  const float e = __expf(-fabsf(dx));
  l = dx > 0.0f ? fmaf(l, e, 1.0f) : l + e;
  m = fmaxf(m, x);
}

// Merges two (max, sum) pairs; an empty pair is (-inf, 0).
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  if (mm != -INFINITY) {
    l = l * __expf(m - mm) + l2 * __expf(m2 - mm);
    m = mm;
  }
}

// Butterfly stage of the query transform across lanes at distance M: the
// lane with bit M clear keeps a + b, its partner a - b (lane holds R values).
template <int M, int R>
__device__ __forceinline__ void qlane_stage(float (&v)[R], int lane) {
  const float sgn = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = fmaf(v[r], sgn, lane_xor<M>(v[r]));
}

// Walsh-Hadamard transform (no scale) of a row spread over a wave, lane l
// holding coordinates l + 64 r: butterflies over r in registers, then over
// the lane bits by cross-lane exchange.
template <int R>
__device__ __forceinline__ void wht_row(float (&v)[R], int lane) {
#pragma unroll
  for (int h = 1; h < R; h <<= 1) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  qlane_stage<1>(v, lane);
  qlane_stage<2>(v, lane);
  qlane_stage<4>(v, lane);
  qlane_stage<8>(v, lane);
  qlane_stage<16>(v, lane);
  qlane_stage<32>(v, lane);
}

// Element r of a row stored as fp32, fp16 or bf16, at lane + 64 r.
__device__ __forceinline__ float row_elem(const void* p, int dtype, size_t i) {
  if (dtype == AXR_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if (dtype == AXR_F16) return __half2float(__ushort_as_half(h));
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Table shapes.  SG = false: int32 fixed-point entries for every field value
// (the mirrored half written by negation).  SG = true: fp32 entries for the
// fields whose top bit is clear only; a field f with the top bit set reads the
// entry of its mirror ~f and negates it (the codebook's symmetry makes the two
// exact negatives), which halves the table so that pairs of 4-bit fields fit.
template <int D, int BITS, int P, bool SG = false>
struct ScoreShape {
  static constexpr int LPK = D / 32;            // lanes per key
  static constexpr int KPG = 16 / LPK;          // keys per 16-lane group
  static constexpr int KPW = 64 / LPK;          // keys per wave
  static constexpr int WL = BITS;               // record words per lane (32 coords)
  static constexpr int W = D * BITS / 32;       // record words per key
  static constexpr int FB = P * BITS;           // field bits per group
  static constexpr int NE = 1 << FB;            // field values per group
  static constexpr int NES = SG ? NE / 2 : NE;  // entries stored per group
  static constexpr int NV = 32 / P;             // groups per lane
  // Sets of NES 256-byte rows: one per 16 groups of a lane chunk.  With
  // fewer than 16 groups per chunk (P = 4), chunk u's groups take the
  // columns (v + KPG u) mod 16, v < NV, and the chunks u, u + RS, ... take
  // disjoint columns, so they share one row set.
  static constexpr int RS = LPK * NV / 16;      // row sets per 4-head table
  static constexpr int TBYTES = 256 * NES * RS;  // bytes per 4-head table
  // first row of the set holding group v of chunk u
  static constexpr int row_base(int u, int v) {
    return NV >= 16 ? (u * (NV / 16) + v / 16) * NES : (u % RS) * NES;
  }
};

constexpr int IL = 1;                // record units processed together
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dword format

// The width-bit field at bit pos of an N-word bit string, moved to bits
// 8 .. 8 + width (other bits are left; the caller masks with
// ((1 << width) - 1) << 8 and ors the result into a table address).
template <int N>
__device__ __forceinline__ uint32_t field_shl8_raw(const uint32_t (&w)[N], int pos, int width) {
  const int wi = pos >> 5, sh = pos & 31;
  if (sh + width <= 32) {
    if (sh >= 8) return w[wi] >> (sh - 8);
    return w[wi] << (8 - sh);
  }
  return __builtin_amdgcn_alignbit(w[(wi + 1) % N], w[wi], sh - 8);
}

// (a & mask) | c in one instruction (the compiler would otherwise emit an and
// and an add for disjoint bits).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
}

// Byte k of x written into byte 1 of a, the other bytes of a kept: one
// v_mov with SDWA selects (k is a compile-time constant after unrolling).
__device__ __forceinline__ void byte_into_byte1(uint32_t& a, uint32_t x, int k) {
  switch (k) {
    case 0:
      asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0"
          : "+v"(a) : "v"(x));
      break;
    case 1:
      asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1"
          : "+v"(a) : "v"(x));
      break;
    case 2:
      asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_2"
          : "+v"(a) : "v"(x));
      break;
    default:
      asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
          : "+v"(a) : "v"(x));
      break;
  }
}

// (byte k of s | byte 0 of c) << 24, zeros elsewhere: with s holding only the
// top bit of each byte and c = 0x3F, the fp32 value +0.5 or -0.5.
__device__ __forceinline__ float half_sign(uint32_t s, uint32_t c, int k) {
  uint32_t r;
  switch (k) {
    case 0:
      asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:BYTE_0 "
          "src1_sel:BYTE_0" : "=v"(r) : "v"(s), "v"(c));
      break;
    case 1:
      asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
          "src1_sel:BYTE_0" : "=v"(r) : "v"(s), "v"(c));
      break;
    case 2:
      asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:BYTE_2 "
          "src1_sel:BYTE_0" : "=v"(r) : "v"(s), "v"(c));
      break;
    default:
      asm("v_or_b32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PAD src0_sel:BYTE_3 "
          "src1_sel:BYTE_0" : "=v"(r) : "v"(s), "v"(c));
      break;
  }
  return __uint_as_float(r);
}

template <int WL>
__device__ __forceinline__ void buffer_load_words(uint32_t (&dst)[WL], __amdgpu_buffer_rsrc_t r,
                                                  uint32_t voff, uint32_t soff) {
  if constexpr (WL == 2) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    dst[0] = v.x; dst[1] = v.y;
  } else if constexpr (WL == 3) {
    typedef uint32_t v3u __attribute__((ext_vector_type(3)));
    const v3u v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z;
  } else {
    static_assert(WL == 4, "2, 3 or 4 record words per lane");
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
}

// What a launch computes besides the scores: nothing, the split-T softmax
// partials, the fused decode step's new key, or (kFused) the records and
// norms of every key it scores, quantized from the raw keys (KDT their
// dtype) in the same pass.
enum ScoreMode { kPlain = 0, kLse = 1, kDecode = 2, kFused = 3 };

template <int D, int BITS, int P, int NT, int NTHREADS, int MODE, bool SG, int KDT = AXR_F16>
__global__ __launch_bounds__(NTHREADS) void score_kernel(const void* __restrict__ q, int qdt,
                                                       const uint32_t* __restrict__ packed,
                                                       const float* __restrict__ norms,
                                                       float* __restrict__ scores,
                                                       ScoreParams prm) {
  using S = ScoreShape<D, BITS, P, SG>;
  static_assert(!SG || (S::LPK == 4 && S::FB == 8),
                "signed half tables are built for 8-bit pair fields at d = 128");
  constexpr int GB = 4 * NT;                    // heads per block (some may be padding)
  constexpr int L = 1 << BITS;                  // codebook levels
  constexpr int HL = L / 2;
  // Static LDS (compile-time offsets fold into the read instructions):
  // NT tables of S::TBYTES bytes, q' [GB][D] and the head scales.
  __shared__ int4 lut[NT * (S::TBYTES / 16)];
  __shared__ float qs[GB][D];
  __shared__ float hinv[GB], hinv2[GB];        // 2^-e of each head's scale, as two exact factors
  __shared__ int4 qterm[P == 4 ? (1 << BITS) * D : 1];  // rounded terms of a 4-coordinate table

  const int tid = threadIdx.x;
  // Block id -> (row, tile, head group).  With several head groups, the
  // blocks of one (row, tile) are 8 ids apart: ids are dealt to the 8 XCDs
  // round-robin, so they run on one XCD and the later reads of the records
  // they share hit its L2.  Ids past the last (row, tile) have no work.
  int tile, hg, row;
  if (prm.head_groups == 1) {
    tile = blockIdx.x % prm.tiles;
    hg = 0;
    row = blockIdx.x / prm.tiles;
  } else {
    const int q8 = blockIdx.x / 8;
    const int rt = (q8 / prm.head_groups) * 8 + blockIdx.x % 8;
    if (rt >= prm.row_tiles) return;
    hg = q8 % prm.head_groups;
    tile = rt % prm.tiles;
    row = rt / prm.tiles;
  }
  const int bi = row / prm.Hkv;
  const int kvh = row % prm.Hkv;
  const int h0 = kvh * prm.G + hg * GB;         // first query head of the block
  const int nvalid = min(GB, prm.G - hg * GB);  // heads of this block that exist
  const int wave = tid / 64, lane = tid % 64;
  const int u = lane % S::LPK;                  // 32-coordinate chunk of the key
  const int kw = lane / S::LPK;                 // key index in the wave
  constexpr uint32_t REC_BYTES = S::W * 4;
  // steps per batch of lookups (quantize-and-score with two tables: two,
  // which keeps its registers near 128; four spilled more and ran 100 µs
  // against 87 µs on the long-context cache)
  constexpr int CH = (MODE == kFused && NT == 2) ? 2 : (8 / NT < S::NV ? 8 / NT : S::NV);
  // record units in flight per wave: the 4-coordinate table's units cost
  // the fewest instructions, so more of them are kept in flight (5 measured
  // fastest, against 3, 4, 6 and 8)
  // (fused: one unit of raw keys in flight; two measured 3.5 % slower, with
  // 128 VGPRs instead of 110)
  constexpr int PD = MODE == kFused ? 1 : (NT == 1 ? (P == 4 ? 5 : 3) : 2);
  // Fused quantize-and-score: a lane loads the raw words of its key's 32
  // coordinates (the write path's layout at d = 128: lane u holds block u
  // and quantizes it into exactly the b record words that it looks up).
  constexpr bool FUSED = MODE == kFused;
  static_assert(!FUSED || (S::LPK == 4 && !SG && BITS <= 3),
                "quantize-and-score is built for d = 128, b = 2 or 3");
  constexpr int KW = FUSED ? RawWords<KDT>::kWords : 4;   // raw words per lane
  constexpr uint32_t KEY_BYTES = D * (KDT == AXR_F32 ? 4u : 2u);
  // tokens [0, len) of this batch row are scored: T, or lens[bi] (clamped),
  // or pos[bi] + 1 in a fused decode step
  int64_t len = prm.T;
  int64_t slot = -1;                            // the decode step's new token
  if constexpr (MODE == kDecode) {
    slot = prm.pos[bi];
    const int64_t l = slot + 1;
    len = l < 0 ? 0 : (l < prm.T ? l : prm.T);
  } else if (prm.lens != nullptr) {
    const int64_t l = prm.lens[bi];
    len = l < 0 ? 0 : (l < prm.T ? l : prm.T);
  }
  const int64_t t0 = static_cast<int64_t>(tile) * prm.tile_len;
  if (t0 >= len) {                              // block-uniform: nothing to score
    if (MODE == kLse && tid < nvalid) {
      float* part = prm.partials + ((static_cast<size_t>(bi) * prm.Hq + h0 + tid) * prm.tiles + tile) * 2;
      part[0] = -INFINITY;
      part[1] = 0.0f;
    }
    return;
  }
  const int64_t t1 = (t0 + prm.tile_len < len) ? t0 + prm.tile_len : len;
  const size_t rowbase = static_cast<size_t>(row) * prm.t_cap;
  // block-uniform: this tile holds the decode step's new token
  const bool holds_new = MODE == kDecode && slot >= t0 && slot < t1;
  // a new token at or past T but inside the cache is scored by no tile; the
  // first head group's block of the row's last tile stores it
  const bool tail_new = MODE == kDecode && slot >= prm.T && slot < prm.t_cap &&
                        tile == prm.tiles - 1 && hg == 0;
  const bool makes_new = holds_new || tail_new;
  __shared__ uint8_t nidx[D];                   // its indices, then its record
  __shared__ uint32_t newrec[S::W];
  __shared__ float newnrm;

  // Records and norms of this (batch, KV head) row through raw buffer
  // resources that end at this block's last token: loads past the tile return
  // 0 without touching memory, so prefetching needs no clamping and fetches
  // nothing beyond the tile.
  const __amdgpu_buffer_rsrc_t rrec = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(packed + rowbase * S::W), 0,
      static_cast<int>(static_cast<uint32_t>(t1) * REC_BYTES), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rnrm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(norms + rowbase), 0, static_cast<int>(static_cast<uint32_t>(t1) * 4u),
      kRsrcWord3);
  // The tile is cut into units of S::KPW tokens, one per wave per batch:
  // unit k holds tokens t0 + k KPW + [0, KPW).  Each wave's first PD units
  // are fixed (the block's first PD batches, wave-interleaved); the rest come
  // from an LDS counter, IL at a time, so the waves that the issue
  // arbitration favours take more of them and all waves end together.  Unit
  // offsets go into the vector offset, which the buffer range check covers.
  constexpr int NW = NTHREADS / 64;
  const uint32_t wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t tile_keys = static_cast<uint32_t>(t1 - t0);
  const uint32_t units = (tile_keys + S::KPW - 1) / S::KPW;
  __shared__ uint32_t next_unit;
  if (tid == 0) next_unit = PD * NW;
  const uint32_t vrec = static_cast<uint32_t>(t0 + kw) * REC_BYTES + u * (S::WL * 4);
  const uint32_t vnrm = static_cast<uint32_t>(t0 + kw) * 4u;
  // Fused: the raw keys of the row, through a resource that ends at the
  // tile's last token (loads past it return zeros, a zero key, whose record
  // is not stored), and the write path's per-lane sign pattern.
  const __amdgpu_buffer_rsrc_t rkey = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(FUSED ? static_cast<const void*>(static_cast<const char*>(prm.keys) +
                                                          rowbase * KEY_BYTES)
                              : static_cast<const void*>(packed)),
      0, static_cast<int>(FUSED ? static_cast<uint32_t>(t1) * KEY_BYTES : 0u), kRsrcWord3);
  const uint32_t vkey = static_cast<uint32_t>(t0 + kw) * KEY_BYTES + u * (KEY_BYTES / S::LPK);
  auto load_raw = [&](uint32_t (&r)[KW], uint32_t unit) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(
          rkey, vkey + unit * (S::KPW * KEY_BYTES) + 16u * i, 0, 0);
      r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
    }
  };

  // 1. q' = H (s * q) / sqrt(d) for head g by wave g, in registers: lane l
  //    holds coordinates l + 64 r; butterflies over r in registers and over
  //    the lane bits by cross-lane exchange.  The same wave sums |q'_j| (in a
  //    fixed order, so every block of a row gets the same scale) and picks
  //    the head's fixed-point scale 2^e with sum_j |q'_j| max|c| 2^e < 2^31:
  //    the sum of a key's table entries then fits int32 (with at most d/2 of
  //    rounding on top, far below the 1e-4 relative slack of the bound), and
  //    the 32-bit sums, which wrap, end exact.
  constexpr int R = D / 64;
  float v[R];
  uint32_t raw[R];
  if (wave < GB) {
    // All loads of the head are issued before the first wait (one memory
    // round trip); the sign words are kernel arguments read at uniform
    // indices, so they come from scalar registers.
    const int g = wave < nvalid ? wave : 0;   // padding heads load head 0, zeroed below
    const size_t qrow = (static_cast<size_t>(bi) * prm.Hq + h0 + g) * D + lane;
    if (qdt == AXR_F32) {
#pragma unroll
      for (int r = 0; r < R; ++r) raw[r] = static_cast<const uint32_t*>(q)[qrow + 64 * r];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) raw[r] = static_cast<const uint16_t*>(q)[qrow + 64 * r];
    }
  }

  // The first PD batches of record loads go out right behind the query loads
  // (which start the critical path and should not queue behind them), so
  // that their memory latency overlaps the query transform and the table
  // build.
  uint32_t wq[PD][S::WL];
  float nq[PD];
  uint32_t rq[FUSED ? PD : 1][KW];              // fused: raw key words in flight
  uint32_t ks[PD];                              // unit of each batch in flight
#pragma unroll
  for (int pd = 0; pd < PD; ++pd) {
    ks[pd] = static_cast<uint32_t>(pd * NW) + wave_s;
    if constexpr (FUSED) {
      load_raw(rq[pd], ks[pd]);
    } else {
      buffer_load_words<S::WL>(wq[pd], rrec, vrec + ks[pd] * (S::KPW * REC_BYTES), 0);
      nq[pd] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             rnrm, vnrm + ks[pd] * (S::KPW * 4u), 0, 0));
    }
  }

  if (wave < GB) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float x;
      if (qdt == AXR_F32) {
        x = __uint_as_float(raw[r]);
      } else if (qdt == AXR_F16) {
        x = __half2float(__ushort_as_half(static_cast<unsigned short>(raw[r])));
      } else {
        x = __uint_as_float(raw[r] << 16);
      }
      const uint32_t s_lo = __builtin_amdgcn_readfirstlane(prm.sign[2 * r]);
      const uint32_t s_hi = __builtin_amdgcn_readfirstlane(prm.sign[2 * r + 1]);
      const uint32_t sw = (lane & 32) ? s_hi : s_lo;
      const uint32_t neg = ((sw >> (lane & 31)) & 1u) << 31;
      v[r] = wave < nvalid ? __uint_as_float(__float_as_uint(x) ^ neg) : 0.0f;
    }
  }
  if (wave < GB) {
    const int g = wave;
    wht_row<R>(v, lane);
    const float inv_sqrt_d = 1.0f / sqrtf(static_cast<float>(D));
    float sa = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      v[r] *= inv_sqrt_d;
      sa += fabsf(v[r]);
    }
    sa += lane_xor<1>(sa);
    sa += lane_xor<2>(sa);
    sa += lane_xor<4>(sa);
    sa += lane_xor<8>(sa);
    sa += lane_xor<16>(sa);
    sa += lane_xor<32>(sa);
    // The butterfly leaves the same sum in every lane (each step adds the
    // same two values, in either order), so every lane picks the same scale
    // and stores its coordinates of q' already multiplied by it (exact: a
    // power of two, applied as two factors that never leave fp32's range).
    const float cmax = fabsf(prm.centroid[L - 1]);
    const float f = sa * cmax * 1.0001f;
    int e = 0;
    if (f > 0.0f) frexpf(f, &e);                // f < 2^e
    int sh = SG ? 0 : 31 - e;                   // fp32 entries need no fixed point
    // up to 2^252 for tiny queries, applied as two powers of two that are
    // each representable (the second is 1 unless sh > 126)
    sh = sh > 252 ? 252 : (sh < -126 ? -126 : sh);
    const int sh1 = sh > 126 ? 126 : sh;
    const float s1 = ldexpf(1.0f, sh1), s2 = ldexpf(1.0f, sh - sh1);
#pragma unroll
    for (int r = 0; r < R; ++r) qs[g][lane + 64 * r] = (v[r] * s1) * s2;
    if (lane == 0) {
      hinv[g] = ldexpf(1.0f, -sh1);
      hinv2[g] = ldexpf(1.0f, sh1 - sh);
    }
  }
  // Fused decode step: one wave quantizes the new key with the write path's
  // rule (sign pattern, Walsh-Hadamard transform, index = number of
  // thresholds below z, a zero key in the cell below 0), lane l holding
  // coordinates l + 64 r; indices go to LDS for packing below.
  if (MODE == kDecode && makes_new && wave == NTHREADS / 64 - 1) {
    const size_t krow = (static_cast<size_t>(bi) * prm.Hkv + kvh) * D + lane;
    float kv[R];
    float ss = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float x = row_elem(prm.knew, prm.kdt, krow + 64 * r);
      ss = fmaf(x, x, ss);
      const uint32_t s_lo = __builtin_amdgcn_readfirstlane(prm.sign[2 * r]);
      const uint32_t s_hi = __builtin_amdgcn_readfirstlane(prm.sign[2 * r + 1]);
      const uint32_t sw = (lane & 32) ? s_hi : s_lo;
      kv[r] = __uint_as_float(__float_as_uint(x) ^ (((sw >> (lane & 31)) & 1u) << 31));
    }
    ss += lane_xor<1>(ss);
    ss += lane_xor<2>(ss);
    ss += lane_xor<4>(ss);
    ss += lane_xor<8>(ss);
    ss += lane_xor<16>(ss);
    ss += lane_xor<32>(ss);
    float nrm = sqrtf(ss);
    wht_row<R>(kv, lane);
    if (!(nrm >= 0x1p-50f && nrm <= 0x1p50f)) {
      // squares that underflow or overflow fp32: the norm again from the
      // transformed coordinates scaled by 2^64 or 2^-64 (exact; the
      // transform scales norms by sqrt(d)), as the write path does
      const bool tiny = !(nrm >= 0x1p-50f);
      const float up = tiny ? 0x1p64f : 0x1p-64f;
      float s2 = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float t = kv[r] * up;
        s2 = fmaf(t, t, s2);
      }
      s2 += lane_xor<1>(s2);
      s2 += lane_xor<2>(s2);
      s2 += lane_xor<4>(s2);
      s2 += lane_xor<8>(s2);
      s2 += lane_xor<16>(s2);
      s2 += lane_xor<32>(s2);
      nrm = (sqrtf(s2) * (tiny ? 0x1p-64f : 0x1p64f)) * (1.0f / sqrtf(static_cast<float>(D)));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float a = fabsf(kv[r]);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i + 1 < HL; ++i) cnt += a > prm.tpos[i] * nrm ? 1 : 0;
      nidx[lane + 64 * r] = static_cast<uint8_t>(kv[r] > 0.0f ? HL + cnt : HL - 1 - cnt);
    }
    if (lane == 0) newnrm = nrm;
  }
  // Fused: the write path's sign masks of the key's four blocks, one LDS row
  // per block (by the waves that hold no query head)
  __shared__ uint4 sgl[FUSED ? S::LPK * KW / 4 : 1];
  if constexpr (FUSED) {
    if (tid >= 64 * GB)
      WhtLane<D, KDT>::fill_sign_masks(reinterpret_cast<uint32_t*>(sgl), prm.sign, tid - 64 * GB,
                                       NTHREADS - 64 * GB);
  }
  __syncthreads();

  // ... and packs them into the record: thread i of the last wave assembles
  // word i; the first head group's block also stores record and norm.
  if (MODE == kDecode && makes_new && tid >= NTHREADS - S::W) {
    const int wi = tid - (NTHREADS - S::W);
    uint32_t word = 0u;
    for (int j = (32 * wi) / BITS; j <= (32 * wi + 31) / BITS && j < D; ++j) {
      const int sh = BITS * j - 32 * wi;
      const uint32_t v = nidx[j];
      word |= sh >= 0 ? v << sh : v >> (-sh);
    }
    newrec[wi] = word;
    if (hg == 0) {
      prm.packed_out[(rowbase + static_cast<size_t>(slot)) * S::W + wi] = word;
      if (wi == 0) prm.norms_out[rowbase + static_cast<size_t>(slot)] = newnrm;
    }
  }

  // 2. the tables, one 16-byte entry (4 heads) per (lane chunk u, group v,
  //    field f).  The codebook is symmetric (c[L-1-k] = -c[k]), so the entry
  //    of the fully mirrored field is the negation: each task rounds the
  //    coordinate terms once and writes an entry and its mirror.  A pair
  //    (or 4-coordinate) entry is the sum of its rounded coordinate terms.
  {
    auto slot_of = [](int uu, int vv, int ff) {
      return 16 * (S::row_base(uu, vv) + ff) + ((vv + S::KPG * uu) & 15);
    };
    constexpr int HALF_NE = S::NE / 2;           // fields with the top bit clear
    constexpr int GROUPS = NT * S::LPK * S::NV;  // (table, chunk, group) triples
    // FSPLIT threads share a triple, each taking every FSPLIT-th field, so a
    // thread reads its coordinates and head scales once.  Triple index
    // fastest: the 16 lanes of a quarter-wave write 16 distinct LDS columns.
    constexpr int FSPLIT = NTHREADS / GROUPS < 1 ? 1
                           : (NTHREADS / GROUPS < HALF_NE ? NTHREADS / GROUPS : HALF_NE);
    static_assert(P != 4 || (BITS == 2 && !SG && NT == 1 && S::LPK == 4),
                  "4-coordinate groups are built for b = 2 at d = 128, one table");
    if constexpr (P == 4) {
      // (a) the rounded coordinate terms q'_j c_k 2^e of the 4 heads, one
      //     16-byte record per (level k, coordinate c of its group, group g)
      //     at ((4 k + c) 32 + g), heads already in chunk g / 8's component
      //     order; (b) each entry the sum of its four terms.  Group index
      //     fastest in both: the 16 lanes of a quarter-wave read 16 columns.
      constexpr int NG = D / 4;                  // groups of a key
      for (int t = tid; t < L * 4 * NG; t += NTHREADS) {
        const int g = t % NG, c = (t / NG) % 4, k = t / (4 * NG);
        const int j = 4 * g + c;
        const int pu = (j / 32) & 3;
        const float ck = prm.centroid[__builtin_amdgcn_readfirstlane(k)];
        int e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __float2int_rn(qs[i ^ pu][j] * ck);
        qterm[t] = make_int4(e[0], e[1], e[2], e[3]);
      }
      __syncthreads();
      for (int item = tid; item < NG * HALF_NE; item += NTHREADS) {
        const int g = item % NG, f = item / NG;  // f: top bit clear
        const int uu = g / S::NV, vv = g % S::NV;
        int4 e = qterm[(4 * (f & 3) + 0) * NG + g];
#pragma unroll
        for (int c = 1; c < 4; ++c) {
          const int4 t = qterm[(4 * ((f >> (2 * c)) & 3) + c) * NG + g];
          e.x += t.x;
          e.y += t.y;
          e.z += t.z;
          e.w += t.w;
        }
        lut[slot_of(uu, vv, f)] = e;
        lut[slot_of(uu, vv, (S::NE - 1) ^ f)] = make_int4(-e.x, -e.y, -e.z, -e.w);
      }
    } else {
    static_assert(GROUPS % 64 == 0, "a wave's 64 items share their field index");
    static_assert(HALF_NE % FSPLIT == 0, "every thread of a triple takes as many fields");
    for (int item = tid; item < GROUPS * FSPLIT; item += NTHREADS) {
      const int vv = item % S::NV;
      const int uu = (item / S::NV) % S::LPK;
      const int t4 = (item / (S::NV * S::LPK)) % NT;
      // wave-uniform, so the centroids below come from the kernel arguments
      const int f0 = __builtin_amdgcn_readfirstlane(item / GROUPS);
      const int j = 32 * uu + P * vv;
      int4* tab = lut + t4 * (S::TBYTES / 16);
      // With four lanes per key, component i of chunk u's entries holds head
      // u ^ i (see quad_reduce_scatter); otherwise heads are in order.  The
      // coordinates are read in that order, q'_j 2^e (stored scaled).
      const int pu = S::LPK == 4 ? (uu & 3) : 0;
      float qc[P][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = 4 * t4 + (i ^ pu);
#pragma unroll
        for (int c = 0; c < P; ++c) qc[c][i] = qs[g][j + c];
      }
      // a fixed trip count, unrolled: the centroid loads of every field go
      // out together instead of one scalar load and wait per entry
#pragma unroll
      for (int k = 0; k < HALF_NE / FSPLIT; ++k) {
        const int f = f0 + k * FSPLIT;
        float cc[P];                              // centroid of each coordinate's index
#pragma unroll
        for (int c = 0; c < P; ++c) cc[c] = prm.centroid[(f >> (BITS * c)) & (L - 1)];
        if constexpr (SG) {
          // fp32 entry: the coordinate terms, rounded, then their sum
          float ef[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ef[i] = mul_rounded(qc[0][i], cc[0]);
#pragma unroll
            for (int c = 1; c < P; ++c) ef[i] += mul_rounded(qc[c][i], cc[c]);
          }
          // stored doubled (exact, and finite: every centroid at d = 128,
          // b = 4 is below 1/4 in magnitude): the loop's sign factor is +-0.5
          tab[slot_of(uu, vv, f)] = make_int4(
              __float_as_int(2.0f * ef[0]), __float_as_int(2.0f * ef[1]),
              __float_as_int(2.0f * ef[2]), __float_as_int(2.0f * ef[3]));
          continue;
        }
        int e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = __float2int_rn(qc[0][i] * cc[0]);
#pragma unroll
          for (int c = 1; c < P; ++c) e[i] += __float2int_rn(qc[c][i] * cc[c]);
        }
        const int fm = (S::NE - 1) ^ f;            // every field mirrored
        tab[slot_of(uu, vv, f)] = make_int4(e[0], e[1], e[2], e[3]);
        tab[slot_of(uu, vv, fm)] = make_int4(-e[0], -e[1], -e[2], -e[3]);
      }
    }
    }
  }

  // per-step table offsets of this lane (independent of the key)
  const int kslot = (lane / S::LPK) % S::KPG;   // key slot in the 16-lane group
  uint32_t boff[S::NV];
#pragma unroll
  for (int st = 0; st < S::NV; ++st) {
    const int vv = (st + kslot) % S::NV;
    boff[st] = static_cast<uint32_t>(
        256 * S::row_base(u, vv) + 16 * ((vv + S::KPG * u) & 15));
  }
  const uint32_t rot = static_cast<uint32_t>(kslot * S::FB);
  const uint32_t fmask = static_cast<uint32_t>(S::NES - 1) << 8;
  // Signed half table: one address register per step, byte 1 rewritten with
  // each key's field (the step offset's byte 1 is bit 15, chunk u's low bit,
  // which the field byte carries as umask), and the constant of half_sign.
  static_assert(!SG || (IL == 1 && S::row_base(1, 0) == 128 && S::NV == 16),
                "signed half tables: 128 rows per chunk, one unit at a time");
  uint32_t sgaddr[S::NV];
#pragma unroll
  for (int st = 0; st < S::NV; ++st) sgaddr[st] = boff[st];
  const uint32_t umask = (u & 1) ? 0x80808080u : 0u;
  const uint32_t c3f = 0x3Fu;
  // Fused: the write path's sign pattern and lane-stage multipliers of the
  // block this lane holds.
  WhtLane<D, KDT> wht;
  if constexpr (FUSED) wht.init(lane_block<S::LPK>(u));
  // Scores of this block's heads through a raw buffer resource (uniform
  // base: the block's first head row); each lane stores head u (and u + 4)
  // at a fixed per-lane offset plus a per-batch scalar offset.
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      scores + (static_cast<size_t>(bi) * prm.Hq + h0) * prm.T, 0,
      static_cast<int>(static_cast<uint32_t>(nvalid) * static_cast<uint32_t>(prm.T) * 4u),
      kRsrcWord3);
  uint32_t vsc[NT];
  float ginv_u[NT], ginv2_u[NT];
#pragma unroll
  for (int t4 = 0; t4 < NT; ++t4) {
    const uint32_t g = static_cast<uint32_t>((4 * t4 + u) % GB);
    vsc[t4] = (g * static_cast<uint32_t>(prm.T) + static_cast<uint32_t>(t0 + kw)) * 4u;
  }
  __syncthreads();
  float ginv[GB], ginv2[GB];                    // 2^-e per head, two factors
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    ginv[g] = hinv[g];
    ginv2[g] = hinv2[g];
  }
#pragma unroll
  for (int t4 = 0; t4 < NT; ++t4) {
    ginv_u[t4] = hinv[(4 * t4 + u) % GB];
    ginv2_u[t4] = hinv2[(4 * t4 + u) % GB];
  }

  // 3. stream the tile, keeping PD units of records (fused: raw keys) in
  //    flight and working on IL of them at once (independent lookups
  //    interleave in the LDS queue).  A unit past the tile end is computed
  //    but not stored.
  // softmax partials of the heads this lane stores: with four lanes per key
  // heads 4 * k + u (k < NT), otherwise head u
  constexpr int NSLOT = S::LPK == 4 ? NT : 1;
  constexpr bool want_lse = MODE == kLse;
  const float lse_scale = prm.scale;
  float sm_m[NSLOT], sm_l[NSLOT];
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
    sm_m[k] = -INFINITY;
    sm_l[k] = 0.0f;
  }

  const char* lut_bytes = reinterpret_cast<const char*>(lut);
  // the next IL units, taken one step before they are needed so that the
  // counter's round trip overlaps the lookups; a wave leaves at its first
  // unit past the tile, and every unit it took later lies past it too
  uint32_t grab = 0u;
  if (lane == 0) grab = atomicAdd(&next_unit, static_cast<uint32_t>(IL));
  for (bool more = true; more;) {
#pragma unroll
    for (int pd0 = 0; pd0 < PD; pd0 += IL) {
      if (ks[pd0] >= units) {                   // wave-uniform
        more = false;
        break;
      }
      const uint32_t kn = __builtin_amdgcn_readfirstlane(grab);
      if (lane == 0) grab = atomicAdd(&next_unit, static_cast<uint32_t>(IL));
      uint32_t w[IL][S::WL];
      float nk[IL];
      uint32_t kc[IL];
#pragma unroll
      for (int il = 0; il < IL; ++il) {
        const int pd = pd0 + il;
        kc[il] = ks[pd];
        if constexpr (FUSED) {
          // quantize the unit's keys exactly as the write kernel does, store
          // their records and norms, and score them from registers
          uint32_t raw[KW];
#pragma unroll
          for (int i = 0; i < KW; ++i) raw[i] = rq[pd][i];
          ks[pd] = kn + il;
          load_raw(rq[pd], ks[pd]);
          float x[32];
          // the row offset through an empty asm keeps the mask reads in the
          // loop (hoisted, they would hold KW registers throughout)
          uint32_t srow = static_cast<uint32_t>(lane_block<S::LPK>(u)) * (KW / 4);
          asm volatile("" : "+v"(srow));
          float nr = wht.transform_lds(raw, x, &sgl[srow]);
          nr = rescued_key_norm<S::LPK>(nr, x, prm.inv_sqrt_d);
          float th[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) th[i] = prm.tpos[i] * nr;
          quantize_lane<BITS>(x, th, w[il]);
          nk[il] = nr;
          const uint32_t tb_rel = kc[il] * S::KPW;
          if (tb_rel + kw < tile_keys) {
            const size_t rowk = rowbase + static_cast<size_t>(t0) + tb_rel + kw;
            uint32_t* dst = prm.packed_out + rowk * S::W + u * BITS;
            if constexpr (BITS == 2) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(w[il][0], w[il][1]);
            } else {
#pragma unroll
              for (int i = 0; i < BITS; ++i) dst[i] = w[il][i];
            }
            if (u == 0) prm.norms_out[rowk] = nr;
          }
          rotate_right<S::WL>(w[il], rot);
          continue;
        }
#pragma unroll
        for (int i = 0; i < S::WL; ++i) w[il][i] = wq[pd][i];
        nk[il] = nq[pd];
        if (MODE == kDecode && holds_new) {
          // the new token's record comes from LDS, not from the cache
          if (t0 + static_cast<int64_t>(kc[il]) * S::KPW + kw == slot) {
#pragma unroll
            for (int i = 0; i < S::WL; ++i) w[il][i] = newrec[u * S::WL + i];
            nk[il] = newnrm;
          }
        }
        ks[pd] = kn + il;
        buffer_load_words<S::WL>(wq[pd], rrec, vrec + ks[pd] * (S::KPW * REC_BYTES), 0);
        nq[pd] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rnrm, vnrm + ks[pd] * (S::KPW * 4u), 0, 0));
        rotate_right<S::WL>(w[il], rot);
      }
      // Signed half table: per record word, the top bit of each field byte
      // (s4) and the entry index of each field (x4): f itself when its top
      // bit is clear, else its mirror ~f, whose top bit is clear.  The byte
      // masks (s4 << 1) - (s4 >> 7) are 0xFF exactly where s4 has 0x80 (no
      // carry crosses a byte; the top byte's wraps modulo 2^32).  Lanes of an
      // odd chunk also set each byte's top bit: it is bit 15 of their table
      // offset, the byte that the field fills.
      uint32_t s4[IL][S::WL], x4[IL][S::WL];
      if constexpr (SG) {
#pragma unroll
        for (int il = 0; il < IL; ++il) {
#pragma unroll
          for (int i = 0; i < S::WL; ++i) {
            s4[il][i] = w[il][i] & 0x80808080u;
            const uint32_t mff = (s4[il][i] << 1) - (s4[il][i] >> 7);
            x4[il][i] = w[il][i] ^ mff ^ umask;
          }
        }
      }

      using Acc = typename std::conditional<SG, float, uint32_t>::type;
      Acc acc[IL][GB];
#pragma unroll
      for (int il = 0; il < IL; ++il)
#pragma unroll
        for (int g = 0; g < GB; ++g) acc[il][g] = Acc(0);
      // The lookups of CH steps are issued before any of their sums, so a
      // wave keeps CH * NT * IL table reads in flight.
#pragma unroll
      for (int st0 = 0; st0 < S::NV; st0 += CH) {
        int4 e[CH][IL][NT];
        float sg[CH][IL];                         // +-0.5: field read directly or mirrored
#pragma unroll
        for (int sc = 0; sc < CH; ++sc) {
#pragma unroll
          for (int il = 0; il < IL; ++il) {
            uint32_t addr;
            if constexpr (SG) {
              // field f = byte k of record word i: its entry index (x4's
              // byte) goes into byte 1 of the step's address register, whose
              // other bytes hold the lane's step offset; a field with the
              // top bit set reads its mirror's entry times -1 (the entries
              // are stored doubled, the sign is +-0.5)
              const int st = st0 + sc;
              const int i = st >> 2, k = st & 3;
              byte_into_byte1(sgaddr[st], x4[il][i], k);
              addr = sgaddr[st];
              sg[sc][il] = half_sign(s4[il][i], c3f, k);
            } else {
              const uint32_t x = field_shl8_raw<S::WL>(w[il], (st0 + sc) * S::FB, S::FB);
              addr = and_or(x, fmask, boff[st0 + sc]);
            }
#pragma unroll
            for (int t4 = 0; t4 < NT; ++t4)
              e[sc][il][t4] = *reinterpret_cast<const int4*>(lut_bytes + addr + t4 * S::TBYTES);
          }
        }
#pragma unroll
        for (int sc = 0; sc < CH; ++sc) {
#pragma unroll
          for (int il = 0; il < IL; ++il) {
#pragma unroll
            for (int t4 = 0; t4 < NT; ++t4) {
              if constexpr (SG) {
                acc[il][4 * t4 + 0] = fmaf(__int_as_float(e[sc][il][t4].x), sg[sc][il], acc[il][4 * t4 + 0]);
                acc[il][4 * t4 + 1] = fmaf(__int_as_float(e[sc][il][t4].y), sg[sc][il], acc[il][4 * t4 + 1]);
                acc[il][4 * t4 + 2] = fmaf(__int_as_float(e[sc][il][t4].z), sg[sc][il], acc[il][4 * t4 + 2]);
                acc[il][4 * t4 + 3] = fmaf(__int_as_float(e[sc][il][t4].w), sg[sc][il], acc[il][4 * t4 + 3]);
              } else {
                acc[il][4 * t4 + 0] += static_cast<uint32_t>(e[sc][il][t4].x);
                acc[il][4 * t4 + 1] += static_cast<uint32_t>(e[sc][il][t4].y);
                acc[il][4 * t4 + 2] += static_cast<uint32_t>(e[sc][il][t4].z);
                acc[il][4 * t4 + 3] += static_cast<uint32_t>(e[sc][il][t4].w);
              }
            }
          }
        }
      }
#pragma unroll
      for (int il = 0; il < IL; ++il) {
        const uint32_t tb_rel = kc[il] * S::KPW;  // the unit's first token past t0
        const int64_t t = t0 + tb_rel + kw;
        const bool valid = tb_rel + kw < tile_keys;
        if constexpr (S::LPK == 4) {
          // lane u of the key ends with head u (and u + 4 when NT = 2)
#pragma unroll
          for (int t4 = 0; t4 < NT; ++t4) {
            const Acc a4[4] = {acc[il][4 * t4], acc[il][4 * t4 + 1], acc[il][4 * t4 + 2],
                               acc[il][4 * t4 + 3]};
            const Acc tot = quad_reduce_scatter(a4);
            float sv;
            if constexpr (SG) {
              sv = nk[il] * tot;
            } else {
              sv = (nk[il] * (static_cast<float>(static_cast<int32_t>(tot)) * ginv_u[t4])) *
                   ginv2_u[t4];
            }
            if (valid && 4 * t4 + u < nvalid) {
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sv), rsc,
                                                    vsc[t4], tb_rel * 4u, 0);
            }
            if (want_lse && valid) lse_push(sm_m[t4], sm_l[t4], mul_rounded(sv, lse_scale));
          }
        } else if constexpr (!SG) {
          // sum over the LPK lanes of the key (exact integer sums)
#pragma unroll
          for (int g = 0; g < GB; ++g) {
            acc[il][g] += lane_xor_u32<1>(acc[il][g]);
            acc[il][g] += lane_xor_u32<2>(acc[il][g]);
            if constexpr (S::LPK >= 8) acc[il][g] += lane_xor_u32<4>(acc[il][g]);
            if constexpr (S::LPK >= 16) acc[il][g] += lane_xor_u32<8>(acc[il][g]);
          }
          if (valid) {
#pragma unroll
            for (int g = 0; g < GB; ++g) {
              if (g % S::LPK == u && g < nvalid) {
                const float sc = static_cast<float>(static_cast<int32_t>(acc[il][g])) * ginv[g];
                const float sv = (nk[il] * sc) * ginv2[g];
                scores[(static_cast<size_t>(bi) * prm.Hq + h0 + g) * prm.T + t] = sv;
                if (want_lse) lse_push(sm_m[0], sm_l[0], mul_rounded(sv, lse_scale));
              }
            }
          }
        }
      }
    }
  }

  // Split-T softmax partials of this tile: merge the lanes that hold the same
  // head (lane bits above the key's LPK lanes), then the waves, through LDS.
  if constexpr (want_lse) {
    __shared__ float red[NTHREADS / 64][GB][2];
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) {
      float m = sm_m[k], l = sm_l[k];
      if constexpr (S::LPK <= 4) lse_merge(m, l, lane_xor<4>(m), lane_xor<4>(l));
      if constexpr (S::LPK <= 8) lse_merge(m, l, lane_xor<8>(m), lane_xor<8>(l));
      lse_merge(m, l, lane_xor<16>(m), lane_xor<16>(l));
      lse_merge(m, l, lane_xor<32>(m), lane_xor<32>(l));
      const int head = S::LPK == 4 ? 4 * k + lane : lane;
      if (lane < S::LPK && head < GB) {
        red[wave][head][0] = m;
        red[wave][head][1] = l;
      }
    }
    __syncthreads();
    if (tid < nvalid) {
      float m = -INFINITY, l = 0.0f;
      for (int w = 0; w < NTHREADS / 64; ++w) lse_merge(m, l, red[w][tid][0], red[w][tid][1]);
      float* part = prm.partials + ((static_cast<size_t>(bi) * prm.Hq + h0 + tid) * prm.tiles + tile) * 2;
      part[0] = m;
      part[1] = l;
    }
  }
}

constexpr int kLdsBudget = 128 * 1024;

template <int D, int BITS, int P, bool SG = false>
constexpr int table_bytes(int NT) { return NT * ScoreShape<D, BITS, P, SG>::TBYTES; }

// Pairs when the pair table fits the LDS budget, else single coordinates.
template <int D, int BITS, int NT>
constexpr int pick_p() { return table_bytes<D, BITS, 2>(NT) <= kLdsBudget ? 2 : 1; }

template <int D, int BITS, int NT>
constexpr bool fits() { return table_bytes<D, BITS, pick_p<D, BITS, NT>()>(NT) <= kLdsBudget; }

// 4-bit pairs at d = 128 as a signed half table (128 KiB for four heads);
// elsewhere the int32 tables of pick_p.
template <int D, int BITS>
constexpr bool signed_pairs() { return D == 128 && BITS == 4; }

// 2-bit indices at d = 128 in groups of four coordinates: 8-bit fields, 256
// entries per group, 128 KiB for four heads (half the lookups of pairs).
template <int D, int BITS>
constexpr bool quad_groups() { return D == 128 && BITS == 2; }

template <int D, int BITS, int NT, bool SG>
int launch_nt(const void* q, int qdt, const uint32_t* packed, const float* norms, int B,
              ScoreParams p, float* scores, hipStream_t s, ScoreParams* plan) {
  constexpr int P = SG ? 2 : (quad_groups<D, BITS>() ? 4 : pick_p<D, BITS, NT>());
  constexpr int tbytes = table_bytes<D, BITS, P, SG>(NT);
  constexpr int bytes = tbytes + 4 * NT * D * 4 + 2 * 4 * NT * 4 +  // + q' + scales
                        (P == 4 ? (1 << BITS) * D * 16 : 0);        // + the rounded terms
  static_assert(tbytes <= kLdsBudget, "table exceeds the LDS budget");
  // 1024-thread blocks, except the single-coordinate two-table case whose
  // registers need 512-thread blocks.
  constexpr int NTHREADS = (P == 1 && NT == 2) ? 512 : 1024;
  static_assert(bytes <= 160 * 1024, "LDS per block exceeded");
  using S = ScoreShape<D, BITS, P, SG>;
  constexpr int KPB = (NTHREADS / 64) * S::KPW;
  p.heads_per_block = 4 * NT;
  p.head_groups = (p.G + 4 * NT - 1) / (4 * NT);
  const int64_t rows = static_cast<int64_t>(B) * p.Hkv * p.head_groups;   // block rows
  const int mode = p.keys != nullptr ? kFused
                  : (p.knew != nullptr ? kDecode : (p.partials != nullptr ? kLse : kPlain));
  // One block per CU, each with one tile: a second resident block would
  // halve the tile over which the table build is spread, and the loop is
  // issue-bound either way.
  const int64_t target = 256;
  int64_t tiles = (target + rows - 1) / rows;
  int64_t tile_len = (p.T + tiles - 1) / tiles;
  // amortise the table build over at least four units per wave; with the
  // keys quantized in the same launch (mode kFused) a unit carries the
  // write path's work too, and one unit per wave keeps short caches spread
  // over more CUs
  const int64_t min_tile = (mode == kFused ? 1 : 4) * KPB;
  if (tile_len < min_tile) tile_len = min_tile;
  tile_len = (tile_len + KPB - 1) / KPB * KPB;
  tiles = (p.T + tile_len - 1) / tile_len;
  p.tiles = static_cast<int>(tiles);
  p.tile_len = tile_len;
  const int64_t row_tiles = static_cast<int64_t>(B) * p.Hkv * tiles;
  // head groups of one (row, tile) 8 block ids apart (see the kernel)
  const int64_t grid = p.head_groups == 1 ? row_tiles
                                          : (row_tiles + 7) / 8 * 8 * p.head_groups;
  if (grid > 0x7FFFFFFF) return static_cast<int>(hipErrorInvalidValue);
  p.row_tiles = static_cast<int>(row_tiles);
  if (plan != nullptr) {                        // planning only: report the tiling
    *plan = p;
    return 0;
  }
  const dim3 g(static_cast<unsigned>(grid)), blk(NTHREADS);
  if (mode == kFused) {
    // every key is quantized by exactly one block: one head group per row
    if (p.head_groups != 1) return static_cast<int>(hipErrorInvalidValue);
    if constexpr (S::LPK == 4 && !SG && BITS <= 3) {
      switch (p.kdt) {
        case AXR_F32:
          hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kFused, SG, AXR_F32>), g,
                             blk, 0, s, q, qdt, packed, norms, scores, p);
          break;
        case AXR_F16:
          hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kFused, SG, AXR_F16>), g,
                             blk, 0, s, q, qdt, packed, norms, scores, p);
          break;
        default:
          hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kFused, SG, AXR_BF16>), g,
                             blk, 0, s, q, qdt, packed, norms, scores, p);
          break;
      }
    } else {
      return static_cast<int>(hipErrorInvalidValue);   // the C ABI rejects these shapes
    }
  } else if (mode == kDecode) {
    hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kDecode, SG>), g, blk, 0, s, q,
                       qdt, packed, norms, scores, p);
  } else if (mode == kLse) {
    hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kLse, SG>), g, blk, 0, s, q, qdt,
                       packed, norms, scores, p);
  } else {
    hipLaunchKernelGGL((score_kernel<D, BITS, P, NT, NTHREADS, kPlain, SG>), g, blk, 0, s, q,
                       qdt, packed, norms, scores, p);
  }
  return static_cast<int>(hipGetLastError());
}

// Eight heads per block when G >= 8 and both tables fit; otherwise four.
// The signed half table and the 4-coordinate table take four heads per
// block (a G = 8 row is two blocks, each reading the records).
template <int D, int BITS>
int launch_b(const void* q, int qdt, const uint32_t* packed, const float* norms, int B,
             const ScoreParams& p, float* scores, hipStream_t s, ScoreParams* plan) {
  if constexpr (signed_pairs<D, BITS>()) {
    return launch_nt<D, BITS, 1, true>(q, qdt, packed, norms, B, p, scores, s, plan);
  } else if constexpr (quad_groups<D, BITS>()) {
    return launch_nt<D, BITS, 1, false>(q, qdt, packed, norms, B, p, scores, s, plan);
  } else {
    if constexpr (fits<D, BITS, 2>()) {
      if (p.G >= 8)
        return launch_nt<D, BITS, 2, false>(q, qdt, packed, norms, B, p, scores, s, plan);
    }
    return launch_nt<D, BITS, 1, false>(q, qdt, packed, norms, B, p, scores, s, plan);
  }
}

template <int D>
int launch_d(const void* q, int qdt, const uint32_t* packed, const float* norms, int B, int b,
             const ScoreParams& p, float* scores, hipStream_t s, ScoreParams* plan) {
  switch (b) {
    case 2: return launch_b<D, 2>(q, qdt, packed, norms, B, p, scores, s, plan);
    case 3: return launch_b<D, 3>(q, qdt, packed, norms, B, p, scores, s, plan);
    default: return launch_b<D, 4>(q, qdt, packed, norms, B, p, scores, s, plan);
  }
}

}  // namespace

int launch_score(const void* q, int q_dtype, const uint32_t* packed, const float* norms, int B,
                 int d, int b, const ScoreParams& p, float* scores, void* stream,
                 ScoreParams* plan) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 128: return launch_d<128>(q, q_dtype, packed, norms, B, b, p, scores, s, plan);
    case 256: return launch_d<256>(q, q_dtype, packed, norms, B, b, p, scores, s, plan);
    default: return launch_d<512>(q, q_dtype, packed, norms, B, b, p, scores, s, plan);
  }
}

}  // namespace axr
