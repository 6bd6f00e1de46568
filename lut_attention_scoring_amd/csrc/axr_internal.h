// Internal interfaces between the C-ABI layer (axr_api.cpp), the host
// codebook solver (axr_codebook.cpp) and the HIP kernels (axr_write.hip,
// axr_score.hip).
#pragma once

#include <stdint.h>

namespace axr {

constexpr int kMaxD = 512;
constexpr int kMaxSignWords = kMaxD / 32;
constexpr int kMaxLevels = 16;  // 2^b for b <= 4
constexpr int kCells = 192;          // cells of the 4-bit quantizer's table
constexpr float kCellMid = 96.0f;    // the cell boundary of the middle threshold

// Lloyd-Max quantizer for N(0, 1/d) in double precision, ascending.
struct Codebook {
  int d = 0, b = 0;
  double centroid[kMaxLevels];
  double threshold[kMaxLevels - 1];
};

// Solves the Lloyd-Max conditions for N(0, 1/d) with 2^b levels (b in 1..4).
void solve_codebook(int d, int b, Codebook* out);

// Cached solution for (d, b); thread-safe.
const Codebook& cached_codebook(int d, int b);

// Kernel-side parameters (passed by value as kernel arguments).
struct WriteParams {
  uint32_t sign[kMaxSignWords];   // sign bits, word j/32 bit j%32
  float tpos[kMaxLevels / 2];     // positive thresholds times sqrt(d), ascending
  float inv_sqrt_d;
  // Append mode (pos != nullptr): key i = bi * Hkv + h is stored at cache row
  // i * t_cap + pos[bi]; keys whose pos lies outside [0, t_cap) are skipped.
  const int32_t* pos;
  int64_t t_cap;
  int Hkv;
  // Comparison transform (kIsoFull / kIsoFast): device float [d/4][2][4],
  // (left, right) unit quaternion of each block of 4 coordinates.
  const float* quats;
  // Cells per unit of z / ||k|| of the 4-bit quantizer's cell table (see
  // the write kernel); 0 for other bit widths, or where no scale fits.
  float cell_k;
  // The table itself when cell_k > 0, filled on the host: for cell c,
  // cells[2c] = the number of signed thresholds -tpos[6], ..., 0, ...,
  // tpos[6] whose position t cell_k + kCellMid (fp32 fused multiply-add)
  // lies below c, cells[2c + 1] = the bits of the first such position at or
  // above c (+inf past the last).
  uint32_t cells[2 * kCells];
};

// Write-path transforms: the method's sign pattern + Walsh-Hadamard, and the
// block-quaternion rotations kept for comparison (full SO(4) or one factor).
enum WriteTransform { kWht = 0, kIsoFull = 1, kIsoFast = 2 };

struct ScoreParams {
  uint32_t sign[kMaxSignWords];
  float centroid[kMaxLevels];     // fp32 centroids, ascending
  int64_t T;                      // tokens scored per row
  int64_t t_cap;                  // tokens allocated per (batch, KV head) row
  int Hq, Hkv, G;                 // query heads, KV heads, Hq / Hkv
  int heads_per_block;            // query heads handled by one block
  int head_groups;                // G / heads_per_block
  int tiles;                      // token tiles per row
  int row_tiles;                  // (batch, KV head) rows times tiles
  int64_t tile_len;               // tokens per tile
  const int32_t* lens;            // optional device [B]: tokens scored per batch row (<= T)
  // Optional split-T softmax partials, [B][Hq][tiles] pairs (m, l): the
  // largest scale * score of the tile and sum over the tile of
  // exp(scale * score - m); (-inf, 0) for a tile with no tokens.
  float* partials;
  float scale;
  // Optional fused decode step (knew != nullptr): the new key knew[bi][kvh]
  // (dtype kdt) is quantized with the write path's rule into slot pos[bi] of
  // the cache (stored by the first head group's block) and row bi is scored
  // for t < pos[bi] + 1 with that record in place.
  const void* knew;
  int kdt;
  const int32_t* pos;
  uint32_t* packed_out;           // the cache (same buffers as packed / norms)
  float* norms_out;
  float tpos[kMaxLevels / 2];     // positive thresholds times sqrt(d)
  // Optional quantize-and-score (keys != nullptr): the raw keys
  // [B][Hkv][T][d] (dtype kdt) are quantized with the write path's rule, their
  // records and norms stored in packed_out / norms_out (t_cap = T) and scored
  // from registers.
  const void* keys;
  float inv_sqrt_d;               // 1 / sqrt(d), as the write path rounds it
};

// Library-held device scratch of axr_score_softmax_noalloc (split-T
// partials), one array per device, and its device address on the current
// device (looked up once per device; returns a hipError_t value as int).
constexpr int64_t kScratchBytes = 1 << 20;
int scratch_address(void** ptr);

// Launchers (return a hipError_t value as int; 0 = success).
int launch_write(const void* keys, int dtype, int64_t n, int d, int b, const WriteParams& p,
                 uint32_t* packed, float* norms, float* y, int mode, void* stream,
                 int tf = kWht);
// With plan != nullptr nothing is launched: *plan receives the parameters
// (tiles, tile_len, head grouping) that a launch with the same sizes uses.
int launch_score(const void* q, int q_dtype, const uint32_t* packed, const float* norms,
                 int B, int d, int b, const ScoreParams& p, float* scores, void* stream,
                 ScoreParams* plan = nullptr);
// Softmax over each score row from the split-T partials: in place,
// scores[bi][h][t] = exp(scale * s - M) / L for t < len(bi), with (M, L) the
// combined partials of the row; lse[bi][h] = M + log L when lse != nullptr.
int launch_softmax(float* scores, const float* partials, const int32_t* lens, int B, int Hq,
                   int64_t T, int tiles, int64_t tile_len, float scale, float* lse,
                   void* stream);

// Sign-pattern selection: exact fp32 scores for rows x Hq x T from keys
// [rows][Hkv][T][d] and q [rows][Hq][d]; per-sample fp64 error sums
// (err[2i] = sum (lut - exact)^2, err[2i+1] = sum exact^2 over `per` scores).
int launch_dense_scores(const void* keys, int kdt, const void* q, int qdt, int rows, int Hq,
                        int Hkv, int64_t T, int d, float* out, void* stream);
// `part` is scratch of score_error_partials(samples) doubles.
int score_error_partials(int samples);
int launch_score_error(const float* lut, const float* exact, int samples, int64_t per,
                       double* part, double* err, void* stream);

// Mode of the write kernel: quantize (indices + norms) or transform export.
enum WriteMode { kWriteQuantize = 0, kWriteTransform = 1, kWriteTransformNormalized = 2 };

}  // namespace axr
