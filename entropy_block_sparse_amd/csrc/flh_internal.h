// Internal interface between the host layer (flh_api.cpp) and the kernels.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "flh.h"

namespace flh {

// Argument checks of a forward call (flh_forward_ex), all but the workspace's.
flh_status forward_check(flh_dtype dt, const void *h, const void *W, const int64_t *targets, int64_t T,
                         int64_t H, int64_t V, const float *logprob, const float *entropy, const float *lse,
                         const flh_active_meta *meta, uint32_t flags);


// Macro tile of every contraction: 256 x 256 outputs per workgroup, 4 waves of
// 128 x 128, K staged 128 bytes at a time (64 bf16 or 32 fp32).
constexpr int kTile = 256;
// Token-tile height of the d-logits skip bitmap; two such tiles form the token
// side of one d-logits workgroup tile.
constexpr int kSkipTile = 128;
// Span pieces: each span is cut into pieces of at most kSpanPiece consecutive rows; a
// hidden-gradient tile takes eight consecutive pieces as its eight 32-row segments.
constexpr int kSpanPiece = 32;
constexpr int kPiecesPerTile = 8;

enum GemmKind : int {
  kFwd = 0,   // z = W h^T tile + online softmax partials          (K = H)
  kDlogits,   // recompute z over active token tiles -> d-logits  (K = H)
  kDhidden,   // dH[span rows] (+)= D[span rows, :] W_s           (K = W_s; B = W^T rows)
  kDweight,   // dW[split rows] = D^T h                          (K = T; A = D^T rows, B = h^T rows)
  kFwdSkip,   // kFwd over pairs of active 128-token tiles only    (K = H)
  kDweightS,  // kDweight times out_scale (bf16 operands widened from fp8 codes of h)
};

// Everything a contraction kernel needs; plain data, passed by value.
struct GemmArgs {
  int64_t T, H, V;
  // vocabulary split (d-logits, dH, dW)
  int64_t v_base;          // first vocabulary row of the split
  int32_t Ws;              // live width of the split
  int32_t ld_d;            // row stride (elements) of the token-major d-logits staging;
                           // columns [0, W_s rounded up to 16 bytes) are written
  // inputs
  const void *h;           // [T, H]
  const void *W;           // [V, H]
  const int64_t *targets;  // [T]
  const float *lse;        // [T]
  const float *entropy;    // [T]
  const float *grad_lp;    // [T] or null
  const float *grad_ent;   // [T] or null
  const uint8_t *mask;     // [T] or null (all active)
  // work lists (backward), device memory
  const int32_t *tile_list;   // token tiles: active ones ascending, then inactive ascending
  const int32_t *counts;      // [0] active token tiles, [1] hidden-gradient tiles, [2] span pieces
  const int32_t *span_tiles;  // span pieces [n][2], half-open token rows
  int32_t n_skip_tiles;       // ceil(T / kSkipTile)
  // outputs / staging
  float *part;             // forward partials [ceil(V/256)][T][4]
  void *D;                 // d-logits staging [T][ld_d]
  void *Dt;                // the same d-logits transposed: [W_s][ld_t]
  const void *Wt;          // this split's rows of W, transposed: [H][ld_wt]
  const void *ht;          // h transposed: [H][ld_t]
  int64_t ld_wt;           // row stride (elements) of Wt, >= W_s (zero padded)
  int64_t ld_t;            // row stride (elements) of ht and Dt, >= T; tokens up to T
                           // rounded up to 16 bytes are written (zeros past T)
  float *dh_acc;           // fp32 hidden-gradient accumulator [T][H]
  int32_t first_split;     // dH: 1 -> overwrite, 0 -> accumulate
  // d-logits: which staging layouts the token-tile pairs with no active token are
  // zero-filled in.  Their d-logits are zero in every split, so the vocabulary-major
  // layout (row stride fixed by T) needs it in the first split only; the token-major
  // layout again whenever its row stride (from the split's live width) changes.
  int32_t zero_tm, zero_vm;
  // Weight gradient over active token tiles only: the vocabulary-major staging and
  // h^T hold just the active 128-token tiles, in the order of the tile list (column
  // 128 r + j is token j of the r-th active tile), and dW contracts over those.
  int32_t compact_dw;
  // Split width the launches and the staging use: the live width W_s, or (the padded
  // baseline the live width replaces, a measurement probe) the widest split's width;
  // operand reads and dW stores stay bounded by W_s.
  int64_t Ws_grid;
  int32_t group_m;         // tiles along M in each rasterization group (the 32 tiles
                           // in flight on one XCD form a group_m x 32/group_m block)
  void *dW;                // [V][H]
  // Logit scale: z = zscale * (accumulated product) in the forward and d-logits
  // epilogues; 1 for bf16 and fp32 inputs, scale_h * scale_w for fp8 inputs (> 0).
  float zscale;
  // Weight-gradient output scale of kDweightS: dW = out_scale * (D^T h^T) with h^T the
  // widened fp8 codes of h, out_scale = scale_h.
  float out_scale;
};

// dtype: 0 = fp32, 1 = bf16 (flh_dtype values), 2 = fp8 E4M3 operands (forward,
// forward over active tiles and d-logits only; their d-logits staging is bf16)
hipError_t launch_gemm(int dtype, GemmKind kind, const GemmArgs &a, int grid, hipStream_t st);

hipError_t launch_spans(const uint8_t *mask, int64_t T, int32_t max_gap, int32_t tile_m,
                        int64_t span_cap, int32_t *spans, int32_t *num_spans,
                        uint32_t *tile_bits, int32_t *active_count, hipStream_t st);

// Work lists of the backward (and of the forward over active tiles: spans NULL, no
// pieces).  Spans are read with their count clamped to [0, span_cap] and each span to
// [0, T].  covered (optional, [ceil(T/32)] words): bit t set iff token t lies inside a
// span and in a token tile whose bit is set.
hipError_t launch_lists(int64_t T, const uint32_t *tile_bits, const int32_t *spans,
                        const int32_t *num_spans, int64_t span_cap, int32_t *tile_list,
                        int32_t *counts, int32_t *span_tiles, int64_t span_tile_cap,
                        hipStream_t st, uint32_t *covered = nullptr);

// Target logits z_y = h[t] . W[y_t] into logprob (NaN for a target outside [0, V)).
// skip_bits: NULL, or the tile bitmap of a forward over active token tiles only (the
// other tiles' tokens are left alone).
// dtype 2: h and W are E4M3 codes, and the dot product of the codes' values is
// multiplied by zscale.
hipError_t launch_target_logit(int dtype, int64_t T, int64_t H, int64_t V, const void *h, const void *W,
                               const int64_t *targets, float *logprob, hipStream_t st,
                               const uint32_t *skip_bits = nullptr, float zscale = 1.f);
// The merge of the per-tile softmax states into lse, entropy and logprob = z_y - lse
// (logprob holds z_y on entry).  skip_bits as above; skipped tokens get 0 for all three.
hipError_t launch_combine(int64_t T, int64_t V, const float *part, float *logprob, float *entropy,
                          float *lse, hipStream_t st, const uint32_t *skip_bits = nullptr);

// Blocked transpose: rows of `in` ([R][C] row-major, elements of esz bytes, 2 or 4)
// are taken in blocks of `block` rows (a multiple of 64; 0 = one block of R rows);
// block b becomes its own [C][ld_out] matrix at out + b * C * ld_out:
// out_b[c][r] = in[b * block + r][c] for rows of the block, and 0 for the rest of
// [0, ld_out).
// Gather form: row_tiles (device, 128-row tiles of `in`) and n_row_tiles (device
// count) set, block = R: output column r = input row row_tiles[r / 128] * 128 + r % 128,
// for r < 128 * n_row_tiles[0] only.
// esz 1: `in` holds E4M3 codes and `out` gets the bf16 values they encode (exact).
hipError_t launch_transpose(int esz, const void *in, int64_t R, int64_t C, void *out, int64_t ld_out,
                            int64_t block, hipStream_t st, const int32_t *row_tiles = nullptr,
                            const int32_t *n_row_tiles = nullptr);

// dh = scale * acc rounded to the output dtype (0 fp32, 1 bf16) for active tokens, +0
// for inactive ones, NaN for active tokens outside `covered` (NULL: every token covered).
hipError_t launch_finalize(int dtype, int64_t T, int64_t H, const float *acc,
                           const uint8_t *mask, const uint32_t *covered, void *dh, hipStream_t st,
                           float scale = 1.f);

}  // namespace flh
