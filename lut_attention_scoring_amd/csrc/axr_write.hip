// Write-path kernels for gfx950: normalise, sign pattern, Walsh-Hadamard
// transform, Lloyd-Max bucketize and bit-pack each key of a KV cache.
//
// "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract:
// an orthogonal transform on write makes every coordinate of a unit key
// close to N(0, 1/d), so a codebook fixed by (d, b) quantizes it; the
// indices are stored once and never dequantized.
//
// Layout: a key of d coordinates is held by LPK = d/32 adjacent lanes, lane u
// owning the 32 coordinates of block blk = lane_block(u) in registers (blk =
// u up to d = 128; beyond, a fixed permutation of the blocks that lets every
// lane stage use DPP).  The transform is five butterfly stages inside each
// lane and log2(LPK) stages across lanes.  The 32 indices of a lane are
// exactly b words of the packed record, so every lane stores its own words
// (at block blk; at d = 128, b = 3 regrouped over the key's four lanes into
// 16-byte stores) and a wave writes one contiguous span.
//
// Lane stages are one fused multiply-add per coordinate, x + m * partner(x):
// inputs of lanes whose block index has an odd number of set bits are
// negated on load (folded into the sign-pattern flip), which makes m = -1
// for the lane with the stage's bit of blk clear and m = +1 for its partner
// and leaves every value un-negated after the last stage.
//
// Quantization compares z = H(s*k) (before the 1/(sqrt(d)||k||) scale)
// against thresholds multiplied by sqrt(d)||k||.  For b = 2 and 3: binary
// search on |z| over the positive thresholds of the symmetric codebook, then
// the mirror image for z <= 0 (a coordinate equal to +0, and every
// coordinate of a zero key, takes the cell just below the middle threshold
// 0); the b index bits of each coordinate are lane masks of compares,
// appended to the record words most significant bit first, one
// add-with-carry per bit.  For b = 4 (fifteen thresholds, where that search
// costs four compares, three selects and four carries per coordinate): a
// table in LDS over uniform cells of z / ||k||, each holding at most one
// threshold, gives the number of thresholds below the coordinate's cell and
// the one inside it, so one compare finishes the index, which is packed a
// nibble at a time.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "axr.h"
#include "axr_device.h"
#include "axr_internal.h"
#include "axr_keyquant.h"

namespace axr {
namespace {

constexpr int kBlock = 256;
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

// Waves per SIMD the compiler is asked to fit at least: 6 (at most 80 VGPRs)
// for the fp16 d = 128 Hadamard kernels with 2 or 3 bits, which once took
// 81-82 VGPRs and ran 5 waves per SIMD (with the sign masks in LDS they take
// ~62 and fit 8 by themselves); the other instances keep the compiler's
// choice (1 sets no bound).
template <int D, int BITS, int DT, int TF>
constexpr int write_waves() {
  return (D == 128 && BITS <= 3 && DT == AXR_F16 && TF == kWht) ? 6 : 1;
}

// TF selects the transform: kWht (sign pattern + Walsh-Hadamard), or the
// block-quaternion comparison transforms kIsoFull / kIsoFast.
template <int D, int BITS, int DT, int TF>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(write_waves<D, BITS, DT, TF>())))
void write_kernel(const void* __restrict__ keys, int64_t n, WriteParams prm,
                  uint32_t* __restrict__ packed, float* __restrict__ norms,
                  float* __restrict__ yout, int mode) {
  constexpr int LPK = D / 32;
  constexpr int KPB = kBlock / LPK;
  constexpr int W = D * BITS / 32;
  constexpr int NW = RawWords<DT>::kWords;
  const int u = threadIdx.x % LPK;
  const int key_in_block = threadIdx.x / LPK;
  // the block of the key this lane loads, transforms and stores
  const int blk = TF == kWht ? lane_block<LPK>(u) : u;
  WhtLane<D, DT> wht;
  if constexpr (TF == kWht) wht.init(blk);
  // the sign masks of every block of a key, one LDS row per block
  __shared__ uint4 sgl[TF == kWht ? LPK * NW / 4 : 1];
  if constexpr (TF == kWht)
    WhtLane<D, DT>::fill_sign_masks(reinterpret_cast<uint32_t*>(sgl), prm.sign, threadIdx.x, kBlock);
  float P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) P[i] = prm.tpos[i];
  // 4-bit quantizer's cell table (cell c: position u in [c, c + 1), with
  // u = z cell_k / ||k|| + kCellMid): the host's table from the kernel
  // arguments, copied to LDS.
  __shared__ uint2 cells[BITS == 4 ? kCells : 1];
  if constexpr (BITS == 4) {
    for (int c = threadIdx.x; c < kCells; c += kBlock)
      cells[c] = make_uint2(prm.cells[2 * c], prm.cells[2 * c + 1]);
  }
  if constexpr (BITS == 4 || TF == kWht) __syncthreads();
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
    const size_t off = static_cast<size_t>(kc) * D + static_cast<size_t>(blk) * 32;

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

    float x[32];
    float nrm;
    if constexpr (TF == kWht) {
      // the row offset through an empty asm: the reads stay in the loop
      // (hoisted, the masks would hold NW registers for the whole kernel)
      uint32_t srow = static_cast<uint32_t>(blk) * (NW / 4);
      asm volatile("" : "+v"(srow));
      nrm = wht.transform_lds(raw, x, &sgl[srow]);
    } else {
      // comparison transform: plain conversion, then the block rotations
      float ss = 0.0f;
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
      nrm = key_norm<LPK>(ss);
#pragma unroll
      for (int k = 0; k < 8; ++k) quat_block<TF == kIsoFull>(&x[4 * k], qa[k], qb[k]);
    }

    nrm = rescued_key_norm<LPK>(nrm, x, prm.inv_sqrt_d);

    if (mode == kWriteQuantize) {
      float S[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) S[i] = P[i] * nrm;
      uint32_t words[BITS];
      if constexpr (BITS == 4) {
        // the cell table where every key of the wave has a norm in
        // [2^-100, 2^100] or 0 (thresholds and cell positions then keep full
        // precision); the threshold search otherwise
        const bool cells_ok = prm.cell_k > 0.0f &&
            (nrm == 0.0f || (nrm >= 0x1p-100f && nrm <= 0x1p100f));
        if (__builtin_amdgcn_ballot_w64(!cells_ok) == 0) {
          const float cells_per_z = nrm > 0.0f ? prm.cell_k / nrm : 0.0f;
          quantize_cells(x, cells_per_z, cells, words);
        } else {
          quantize_lane<BITS>(x, S, words);
        }
      } else {
        quantize_lane<BITS>(x, S, words);
      }
      // b = 3 at d = 128: lane u of a key holds block u, i.e. record words
      // 3u .. 3u + 2; the key's 12 words are regrouped over its four lanes
      // so that lanes 0, 1, 2 each store 16 bytes (words 4u .. 4u + 3),
      // taking the rest from the next lane (DPP quad_perm [1,2,3,3]).  At
      // d = 256 and 512, where this kernel's issue is the limit, the same
      // regrouping measured ~2.5 % slower and a lane stores its 3 words.
      uint32_t rg[4] = {0u, 0u, 0u, 0u};
      if constexpr (BITS == 3 && LPK == 4) {
        uint32_t nx[3];
#pragma unroll
        for (int i = 0; i < 3; ++i)
          nx[i] = static_cast<uint32_t>(
              __builtin_amdgcn_mov_dpp(static_cast<int>(words[i]), 0xF9, 0xF, 0xF, false));
        rg[0] = u == 0 ? words[0] : (u == 1 ? words[1] : words[2]);
        rg[1] = u == 0 ? words[1] : (u == 1 ? words[2] : nx[0]);
        rg[2] = u == 0 ? words[2] : (u == 1 ? nx[0] : nx[1]);
        rg[3] = u == 0 ? nx[0] : (u == 1 ? nx[1] : nx[2]);
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
        uint32_t* dst = packed + static_cast<size_t>(row) * W + blk * BITS;
        if constexpr (BITS == 2) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else if constexpr (BITS == 4) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        } else if constexpr (LPK == 4) {
          if (u < 3)
            *reinterpret_cast<uint4*>(packed + static_cast<size_t>(row) * W + 4 * u) =
                make_uint4(rg[0], rg[1], rg[2], rg[3]);
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
                                                static_cast<size_t>(blk) * 32);
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
  // Two batches of keys per block: a measured optimum on every workload
  // shape between one batch per block (block start-up dominates) and a
  // capped grid of long-running blocks (uneven finish at the end).
  int64_t blocks = (need + 1) / 2;
  if (blocks > (int64_t{1} << 30)) blocks = int64_t{1} << 30;   // the loop covers the rest
  const int grid = static_cast<int>(blocks);
  if (grid == 0) return 0;
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
