// The four contractions of the fused LM head on CDNA4 matrix cores (gfx950).
//
//   forward   z^T = W h^T per (256 vocab x 256 token) tile, K = H, with the online
//             log-softmax statistics reduced in the epilogue (fused linear
//             log-prob and entropy: SkyRL #2376 "What does this PR do?" and the
//             stack's "fuse LM-head entropy for RL" layer).
//   d-logits  the same product recomputed for one vocabulary split over pairs of
//             active 128-token tiles only, with the d-logits of log-prob and
//             entropy formed in the epilogue and stored to the split's
//             live-width staging buffer, token-major and vocabulary-major ("How it
//             works": only active d-logits tiles are processed; the final split
//             allocates its live width).
//   dHidden   D[span rows, :] W_s, accumulated in fp32 across splits, over
//             span-local row tiles only (Gemini "Code Review": d_hidden +=
//             split_d_logits @ split_weight; "How it works": spans, no token
//             reordering).  W_s is read from W^T so that its contraction index is
//             contiguous in memory.
//   dWeight   D^T h over all tokens, dense ("How it works": weight gradients stay
//             a dense contraction), read from the vocabulary-major staging and h^T.
//
// One kernel template serves all four.  A workgroup of 4 waves owns a 256 x 256
// output tile; each wave a 128 x 128 quadrant as 8 x 8 blocks of 16 x 16 MFMA
// accumulators.  Every operand is a set of rows with the contraction index K
// contiguous in memory (h, W, W^T, h^T and the two staging layouts), so there is a
// single load path.  Workgroups are persistent (grid = compute units) and walk a
// tile list whose order keeps the tiles of one XCD (workgroup id mod 8) in a
// compact block, so operand rows are shared in that XCD's L2.
//
// bf16 main loop: operands go straight from global memory into two LDS stages of 64
// K elements (buffer_load ... lds), bounded by buffer descriptors so that rows past
// an operand's end read as zero; the LDS fragment reads of the next K step are
// interleaved with the current step's v_mfma_f32_16x16x32_bf16.  fp32 main loop
// (small problems): register-staged loads into two padded LDS stages, four
// v_mfma_f32_16x16x4_f32 per fragment.
//
// Why 16 x 16 blocks: with random operands the matrix cores run into the chip's power
// limit, and the 16 x 16 x 32 instruction reads and writes half the accumulator bytes
// per flop of the 32 x 32 x 16 one; a register-only loop of it sustains a higher clock
// at the same operand bytes per flop.
#include <hip/hip_runtime.h>

#include "flh_internal.h"

namespace flh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
// fp32 path: two stages of 128 bytes of K per row, rows padded to 144 bytes
constexpr int kRowBytes = 144;
constexpr int kOpBytes = kTile * kRowBytes;  // one operand tile, one stage
constexpr int kLdsBytes = 4 * kOpBytes;      // A and B, two stages (147456 B)
// bf16 path: two stages of 64 K elements (128 bytes per row) per operand
constexpr int kOpStage = kTile * 128;     // one operand, one stage: 32 KiB
constexpr int kStage = 2 * kOpStage;      // 64 KiB
constexpr int kLdsBytesV2 = 2 * kStage + 1024;  // 128 KiB + the prefetch scratch
constexpr int kPfLds = 2 * kStage;                // prefetch scratch: 256 bytes per wave
// bf16 d-logits epilogue: the 256 x 256 tile staged token-major in LDS, rows padded to
// 528 bytes (16-byte aligned, consecutive rows 4 banks apart)
constexpr int kLsPitch = 528;
constexpr int kLdsBytesDlg = kTile * kLsPitch > kLdsBytesV2 ? kTile * kLsPitch : kLdsBytesV2;
// bf16 hidden-gradient epilogue: half a tile of fp32 staged per wave, 32 groups of
// 4 x 256 bytes (one row block, one column block) each padded by 64 bytes
constexpr int kDhGroup = 4 * 256 + 64;
constexpr int kDhWave = 32 * kDhGroup;
constexpr int kLdsBytesDh = 4 * kDhWave > kLdsBytesV2 ? 4 * kDhWave : kLdsBytesV2;

// Shared memory of one kernel instantiation: the main loop's stages plus whatever its
// epilogue stages.
template <typename T, int KIND>
constexpr int lds_bytes() {
  return sizeof(T) == 4 ? kLdsBytes
                        : (KIND == kDlogits || KIND == kDweight || KIND == kDweightS ? kLdsBytesDlg
                                                                : (KIND == kDhidden ? kLdsBytesDh : kLdsBytesV2));
}
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T> struct Elt;
template <> struct Elt<uint8_t> { static constexpr int kPer = 16; };  // OCP E4M3 codes
template <> struct Elt<uint16_t> { static constexpr int kPer = 8; };  // bf16 bit patterns
template <> struct Elt<float> { static constexpr int kPer = 4; };

__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

// Values that are the same in every lane but that the compiler cannot prove so (loads
// through pointers held in the argument struct): taking lane 0's copy puts them in
// scalar registers, so buffer descriptors built from them need no per-lane loop.
__device__ __forceinline__ int64_t uni(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const char *uni(const char *p) {
  return reinterpret_cast<const char *>(uni((int64_t)reinterpret_cast<uintptr_t>(p)));
}

// ---- matrix-core step: acc += a * b for one 16-byte fragment per lane ---------------
// Lane l feeds row (l % 16) of A and column (l % 16) of B with the K elements of
// the 16-byte chunk at position (l / 16) of a 64-byte K slice; A and B use the same
// lane -> K assignment, so every K element is paired with itself.  The 16 x 16
// result: lane l holds column (l % 16), rows 4 (l / 16) .. + 3.
//
// run() is the compiler's builtin, for which the compiler inserts the wait states the
// matrix-core pipeline requires.  run_in_place() (bf16 main loop) issues the same
// instruction from inline assembly with the accumulator tied in place: with the
// builtin, 64 accumulators of 4 registers fill the 256 accumulator registers exactly
// and the register allocator rotates some of them through spare registers on every
// stage, which costs moves and wait states in the loop.  The compiler does not track
// wait states around inline assembly; the bf16 kernels are checked for them on the
// host after compilation, and the last K stage of every tile uses run() so that the
// compiler again owns the hazards of the epilogue that reads the accumulators.
template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
  static __device__ __forceinline__ void run(f32x4 &c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void run_in_place(f32x4 &c, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x4 &c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void run_in_place(f32x4 &c, u32x4 a, u32x4 b) { run(c, a, b); }
};

// x combined with its value in lane l ^ 16 (resp. l ^ 32) under a symmetric operation,
// through the in-register lane swaps of gfx950: v_permlane16_swap (32_swap) of x with
// itself leaves, in every lane, x of the lower and of the upper lane of the pair.  (A
// shuffle would take an LDS round trip per step.)
__device__ __forceinline__ void lanes_x16(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void lanes_x32(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_over_x16_x32(float x) {
  float a, b;
  lanes_x16(x, a, b);
  lanes_x32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_over_x16_x32(float x) {
  float a, b;
  lanes_x16(x, a, b);
  lanes_x32(a + b, a, b);
  return a + b;
}

// Two floats rounded to bf16 (to nearest, ties to even), lo in bits 0..15: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
__device__ __forceinline__ void store4(uint16_t *p, float a, float b, float c, float d) {
  u32x2 v;
  v.x = bf16x2_rne(a, b);
  v.y = bf16x2_rne(c, d);
  *reinterpret_cast<u32x2 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store1(uint16_t *p, float a) { *p = (uint16_t)bf16x2_rne(a, 0.f); }
__device__ __forceinline__ void store1(float *p, float a) { *p = a; }
// 16-byte streaming store (nontemporal): for the d-logits staging of a split (a GiB at
// the Llama-3-8B-like shape, far more than L2), written once and read by the next two
// launches.  (For the weight gradient, measured slower than plain stores.)
__device__ __forceinline__ void store16_nt(char *p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Merge two (max, sum exp(z - max), sum exp(z - max)(z - max)) states.
__device__ __forceinline__ void merge_state(float &M, float &s, float &u, float M2, float s2,
                                            float u2) {
  const float Mn = fmaxf(M, M2);
  if (Mn == kNegInf) return;
  const bool e1 = (M == kNegInf), e2 = (M2 == kNegInf);
  const float c1 = e1 ? 0.f : __expf(M - Mn);
  const float c2 = e2 ? 0.f : __expf(M2 - Mn);
  const float u1n = e1 ? 0.f : c1 * (u + s * (M - Mn));
  const float u2n = e2 ? 0.f : c2 * (u2 + s2 * (M2 - Mn));
  s = (e1 ? 0.f : s * c1) + (e2 ? 0.f : s2 * c2);
  u = u1n + u2n;
  M = Mn;
}

// Position of linear tile id L in an (m_tiles x n_tiles) grid walked in groups of
// GM m-tiles, m fastest: 32 consecutive ids form a GM x 32/GM block.
__device__ __forceinline__ void group_map(int64_t L, int64_t m_tiles, int64_t n_tiles, int64_t GM,
                                          int64_t &mi, int64_t &ni) {
  const int64_t per_group = GM * n_tiles;
  const int64_t g = L / per_group;
  const int64_t r = L - g * per_group;
  const int64_t first = g * GM;
  const int64_t gm = (m_tiles - first) < GM ? (m_tiles - first) : GM;
  mi = first + r % gm;
  ni = r / gm;
}

// One operand tile: 256 rows with K contiguous, ldb bytes apart, in eight segments of
// 32 rows: tile rows [32 j, 32 j + 32) are segment j, whose n (0..32) memory rows start
// at base; tile rows past n read as zero.  Wave w loads segments 2w and 2w+1.  Either
// the tile is two halves, rows [0, 128) the first n0 (<= 128) rows at b0 and rows
// [128, 256) the first n1 rows at b1; or (`pieces` set) segment j is span piece p0 + j
// of the table of (first, end) token pairs, rows of b0, and empty past n_pieces.
// Segments are computed, not stored: an array indexed by the wave number would be
// spilled to scratch memory.
struct RowSrc {
  const char *b0, *b1;
  int64_t n0, n1, ldb;
  const int32_t *pieces;
  int64_t p0, n_pieces;
};
// n_rows consecutive rows from b
__device__ __forceinline__ RowSrc rows_of(const char *b, int64_t n_rows, int64_t ldb) {
  const int64_t n0 = n_rows < 128 ? n_rows : 128;
  return RowSrc{b, b + 128 * ldb, n0, n_rows - n0, ldb, nullptr, 0, 0};
}
// tile rows [0, 128) from b0 (n0 rows), [128, 256) from b1 (n1 rows)
__device__ __forceinline__ RowSrc rows_of2(const char *b0, int64_t n0, const char *b1, int64_t n1,
                                           int64_t ldb) {
  return RowSrc{b0, b1, n0 < 128 ? n0 : 128, n1 < 128 ? n1 : 128, ldb, nullptr, 0, 0};
}
// first token and length of span piece pc (no rows past the last piece)
__device__ __forceinline__ void piece(const int32_t *pieces, int64_t pc, int64_t n_pieces, int64_t &start,
                                      int64_t &len) {
  start = 0;
  len = 0;
  if (pc < n_pieces) {
    start = uni(pieces[2 * pc]);
    len = uni(pieces[2 * pc + 1]) - start;
  }
}
// segment j (wave-uniform) of a tile; kPieces says which form s has
template <bool kPieces>
__device__ __forceinline__ void seg(const RowSrc &s, int j, const char *&base, int64_t &n) {
  if constexpr (kPieces) {
    int64_t st;
    piece(s.pieces, s.p0 + j, s.n_pieces, st, n);
    base = s.b0 + st * s.ldb;
  } else {
    const bool h1 = j >= 4;
    const int64_t r = 32 * (j & 3), nh = (h1 ? s.n1 : s.n0) - r;
    base = (h1 ? s.b1 : s.b0) + r * s.ldb;
    n = nh < 0 ? 0 : (nh > 32 ? 32 : nh);
  }
}

template <typename T, int KIND>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    const GemmArgs a) {
  constexpr bool kF8 = sizeof(T) == 1;  // fp8 (OCP E4M3) operands, 16 x 16 x 128 MFMA
  constexpr bool kV2 = sizeof(T) <= 2;  // bf16 and fp8: LDS-direct ring; fp32: register-staged
  __shared__ __attribute__((aligned(16))) char smem[lds_bytes<T, KIND>()];
  constexpr int kPer = Elt<T>::kPer;    // operand elements per 16-byte chunk
  constexpr int64_t kEsz = sizeof(T);
  // d-logits staging element: the input dtype, except bf16 for fp8 inputs
  using TS = typename std::conditional<kF8, uint16_t, T>::type;
  constexpr int kSPer = Elt<TS>::kPer;
  constexpr int64_t kSEsz = sizeof(TS);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---------------- extents of this launch ----------------
  int64_t m_tiles, n_tiles, K;
  int64_t n_pairs_gemm = 0, n_pairs_all = 0;
  if constexpr (KIND == kFwd) {
    m_tiles = cdiv(a.V, kTile);
    n_tiles = cdiv(a.T, kTile);
    K = a.H;
  } else if constexpr (KIND == kFwdSkip) {
    m_tiles = cdiv(a.V, kTile);
    n_tiles = cdiv(uni(a.counts[0]), 2);  // pairs of active token tiles
    K = a.H;
  } else if constexpr (KIND == kDlogits) {
    m_tiles = cdiv(a.Ws_grid, kTile);
    n_pairs_gemm = cdiv(uni(a.counts[0]), 2);
    n_pairs_all = (a.zero_tm || a.zero_vm) ? cdiv(a.n_skip_tiles, 2) : n_pairs_gemm;
    n_tiles = n_pairs_gemm;
    K = a.H;
  } else if constexpr (KIND == kDhidden) {
    m_tiles = uni(a.counts[1]);
    n_tiles = cdiv(a.H, kTile);
    K = a.Ws_grid;
  } else {
    m_tiles = cdiv(a.Ws_grid, kTile);
    n_tiles = cdiv(a.H, kTile);
    K = a.compact_dw ? (int64_t)uni(a.counts[0]) * kSkipTile : a.T;
  }
  const int64_t n_gemm = m_tiles * n_tiles;
  const int64_t n_items =
      n_gemm + (KIND == kDlogits ? m_tiles * (n_pairs_all - n_pairs_gemm) : 0);
  const int64_t G = gridDim.x;
  const bool remap = (G % 8) == 0;
  // Group height of the rasterization: 8 tiles along M, an 8 x 4 block per XCD.  (4 x 8
  // blocks for the hidden and weight gradients were 2% faster on the Llama-3-8B-like head on
  // one box, equal on another, and 12-19% slower on the stress shape, whose 28 column tiles
  // do not divide into blocks of 8.)
  constexpr int kGroupM = 8;

  const char *hp = reinterpret_cast<const char *>(a.h);
  const char *Wp = reinterpret_cast<const char *>(a.W);
  const char *Dp = reinterpret_cast<const char *>(a.D);

  for (int64_t item = blockIdx.x; item < n_items; item += G) {
    // ---------------- d-logits of token-tile pairs with no active token ----------------
    if constexpr (KIND == kDlogits) {
      if (item >= n_gemm) {
        const int64_t z = item - n_gemm;
        const int64_t mi = z % m_tiles;
        const int64_t p = n_pairs_gemm + z / m_tiles;
        const int64_t c0 = mi * kTile;
        const int64_t c1 = imin(c0 + kTile, cdiv(a.Ws_grid, kSPer) * kSPer);
        // token-major staging: rows of the pair's tokens, columns [c0, c1)
        constexpr int kChunks = kTile / kSPer;
        char *Dw = const_cast<char *>(Dp);
        for (int idx = tid; a.zero_tm && idx < kTile * kChunks; idx += kThreads) {
          const int row = idx / kChunks;
          const int ch = idx - row * kChunks;
          const int64_t e = 2 * p + (row >> 7);
          if (e >= a.n_skip_tiles) continue;
          const int64_t t = (int64_t)a.tile_list[e] * kSkipTile + (row & 127);
          const int64_t col = c0 + (int64_t)ch * kSPer;
          if (t < a.T && col < c1)
            store16_nt(Dw + (t * a.ld_d + col) * kSEsz, u32x4{0u, 0u, 0u, 0u});
        }
        // vocabulary-major staging: rows v in [c0, min(c0 + 256, Ws)), the pair's
        // tokens including the zero padding up to a whole 16-byte chunk
        const int64_t v1 = imin(c0 + kTile, (int64_t)a.Ws);
        constexpr int kVecTile = kSkipTile / kSPer;  // 16-byte vectors per token tile
        char *Dtw = reinterpret_cast<char *>(a.Dt);
        for (int idx = tid; a.zero_vm && idx < kTile * 2 * kVecTile; idx += kThreads) {
          const int vr = idx / (2 * kVecTile);
          const int rem = idx - vr * 2 * kVecTile;
          const int half = rem / kVecTile, vec = rem - half * kVecTile;
          const int64_t e = 2 * p + half;
          const int64_t v = c0 + vr;
          if (e >= a.n_skip_tiles || v >= v1) continue;
          const int64_t t = (int64_t)a.tile_list[e] * kSkipTile + vec * kSPer;
          if (t < cdiv(a.T, kSPer) * kSPer)
            store16_nt(Dtw + (v * a.ld_t + t) * kSEsz, u32x4{0u, 0u, 0u, 0u});
        }
        continue;
      }
    }

    // ---------------- tile coordinates ----------------
    // Workgroups are dealt to the 8 XCDs round-robin (XCD = id mod 8).  Within each
    // round of G tiles, give the workgroups of XCD x a contiguous run of tile ids, so
    // the tiles resident on one XCD form a compact block sharing operand rows in its
    // L2.  The last round may be partial: its n_round tiles are split the same way.
    int64_t L = item;
    if (remap) {
      const int64_t r = item / G;
      const int64_t b = item - r * G;
      const int64_t n_round = imin(G, n_gemm - r * G);
      const int64_t x = b & 7, q = n_round >> 3, rem8 = n_round & 7;
      L = r * G + x * q + imin(x, rem8) + (b >> 3);
    }
    int64_t mi, ni;
    group_map(L, m_tiles, n_tiles, a.group_m > 0 ? a.group_m : kGroupM, mi, ni);

    if constexpr (KIND == kDweight || KIND == kDweightS) {
      if (K == 0) {  // weight gradient over no active token tile (compact form): zeros
        const int64_t v_tile = mi * kTile, n_tile = ni * kTile;
        const int n_rows = (int)imin(a.Ws - v_tile, kTile), n_cols = (int)imin(a.H - n_tile, kTile);
        char *zb = reinterpret_cast<char *>(a.dW) + ((a.v_base + v_tile) * a.H + n_tile) * kEsz;
        constexpr int kCh = kTile / kPer;  // 16-byte chunks per tile row
        for (int idx = tid; idx < kTile * kCh; idx += kThreads) {
          const int r = idx / kCh, c = (idx - r * kCh) * kPer;
          if (r < n_rows && c < n_cols)
            *reinterpret_cast<u32x4 *>(zb + ((int64_t)r * a.H + c) * kEsz) = u32x4{0u, 0u, 0u, 0u};
        }
        continue;
      }
    }

    // ---------------- operand rows ----------------
    RowSrc srcA, srcB;
    if constexpr (KIND == kFwd) {
      const int64_t v0 = mi * kTile, t0 = ni * kTile, ldb = a.H * kEsz;
      srcA = rows_of(Wp + v0 * ldb, a.V - v0, ldb);
      srcB = rows_of(hp + t0 * ldb, a.T - t0, ldb);
    } else if constexpr (KIND == kFwdSkip) {
      // the pair's tiles: active tiles 2 ni and 2 ni + 1 of the list (the second may not exist)
      const int64_t v0 = mi * kTile, ldb = a.H * kEsz;
      srcA = rows_of(Wp + v0 * ldb, a.V - v0, ldb);
      const int64_t e1 = 2 * ni + 1;
      const int64_t tile0 = uni(a.tile_list[2 * ni]);
      const int64_t tile1 = (e1 < uni(a.counts[0])) ? uni(a.tile_list[e1]) : -1;
      srcB = rows_of2(hp + tile0 * kSkipTile * ldb, a.T - tile0 * kSkipTile,
                      hp + (tile1 >= 0 ? tile1 : tile0) * kSkipTile * ldb,
                      tile1 >= 0 ? a.T - tile1 * kSkipTile : 0, ldb);
    } else if constexpr (KIND == kDlogits) {
      const int64_t v0 = mi * kTile, ldb = a.H * kEsz;
      const char *wb = Wp + (a.v_base + v0) * ldb;
      srcA = rows_of(wb, a.Ws - v0, ldb);
      const int64_t e1 = 2 * ni + 1;
      const int64_t tile0 = uni(a.tile_list[2 * ni]);
      const int64_t tile1 = (e1 < a.n_skip_tiles) ? uni(a.tile_list[e1]) : -1;
      srcB = rows_of2(hp + tile0 * kSkipTile * ldb, a.T - tile0 * kSkipTile,
                      hp + (tile1 >= 0 ? tile1 : tile0) * kSkipTile * ldb,
                      tile1 >= 0 ? a.T - tile1 * kSkipTile : 0, ldb);
    } else if constexpr (KIND == kDhidden) {
      // the tile's eight 32-row segments are span pieces 8 mi .. 8 mi + 7 (a piece is at
      // most 32 consecutive rows of one span) of the token-major staging
      const int64_t ldb = (int64_t)a.ld_d * kEsz;
      srcA = RowSrc{Dp, Dp, 0, 0, ldb, a.span_tiles, 8 * mi, uni(a.counts[2])};
      // rows n (hidden units) of this split's block of W^T
      const int64_t n0 = ni * kTile, ldw = a.ld_wt * kEsz;
      const char *wt = reinterpret_cast<const char *>(a.Wt) + n0 * ldw;
      srcB = rows_of(wt, a.H - n0, ldw);
    } else {
      // vocabulary-major staging rows v and h^T rows n, both over all tokens
      const int64_t v0 = mi * kTile, n0 = ni * kTile, ldt = a.ld_t * kEsz;
      const char *dt = reinterpret_cast<const char *>(a.Dt) + v0 * ldt;
      const char *ht = reinterpret_cast<const char *>(a.ht) + n0 * ldt;
      srcA = rows_of(dt, a.Ws - v0, ldt);
      srcB = rows_of(ht, a.H - n0, ldt);
    }

    // acc[i][j][x]: tile row wm * 128 + 16 i + 4 (lane / 16) + x, tile column
    // wn * 128 + 16 j + lane % 16
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[i][j][x] = 0.f;
    if constexpr (KIND == kDhidden && !kV2) {
      // fp32: splits after the first continue the fp32 sum of the earlier splits: start
      // the accumulators from it, so the epilogue is a plain store.  (The bf16 epilogue
      // adds the earlier sum while it stores.)
      if (!a.first_split) {
        const int64_t n_tile = ni * kTile;
        const int n_cols = (int)imin(a.H - n_tile, kTile);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // tile rows wm * 128 + 16 i + .. are rows 16 (i % 2) + .. of piece 4 wm + i / 2
          int64_t pst, pln;
          piece(a.span_tiles, 8 * mi + 4 * wm + (i >> 1), uni(a.counts[2]), pst, pln);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int lr = 16 * (i & 1) + 4 * (lane >> 4) + x;
            const bool ok = lr < pln;
            const float *prow = a.dh_acc + (ok ? pst + lr : 0) * a.H + n_tile;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int col = wn * 128 + (lane & 15) + j * 16;
              acc[i][j][x] = (ok && col < n_cols) ? prow[col] : 0.f;
            }
          }
        }
      }
    }

    if constexpr (!kV2) {
      // ================= fp32: register-staged loads, two padded LDS stages =================
      constexpr int kBK = 128 / sizeof(T);  // K elements per stage
      const int nk = (int)cdiv(K, kBK);
      const bool has_tail = (K % kBK) != 0;
      // Thread owns 16-byte chunk (tid & 7) of tile rows (tid >> 3) + 32 i.  Rows past
      // an operand's end are clamped onto its last valid row: their products reach
      // only outputs that are never stored.
      const int r_base = tid >> 3;
      // (tile row r_base + 32 i is row r_base of segment i; an empty segment reads
      // segment 0's first row)
      auto offsets = [&](auto pieces, const RowSrc &s, uint32_t (&off)[8], const char *(&bp)[8]) {
        const char *b_first;
        int64_t n_first;
        seg<decltype(pieces)::value>(s, 0, b_first, n_first);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const char *bi;
          int64_t ni_;
          seg<decltype(pieces)::value>(s, i, bi, ni_);
          const bool has = ni_ > 0;
          int64_t lr = has ? r_base : 0;
          const int64_t nsg = has ? ni_ : n_first;
          lr = lr < nsg - 1 ? lr : nsg - 1;
          bp[i] = has ? bi : b_first;
          off[i] = (uint32_t)(lr * s.ldb + (tid & 7) * 16);
        }
      };
      uint32_t a_off[8], b_off[8];
      const char *a_bp[8], *b_bp[8];
      offsets(std::integral_constant<bool, KIND == kDhidden>{}, srcA, a_off, a_bp);
      offsets(std::false_type{}, srcB, b_off, b_bp);
      // this thread's chunk of K stage kt lies (at least partly) inside K
      auto chunk_in = [&](int kt) -> bool {
        return !(has_tail && kt == nk - 1) || ((int64_t)kt * kBK + (tid & 7) * kPer < K);
      };
      auto load_rows = [&](const char *const (&bp)[8], const uint32_t (&off)[8], int kt, u32x4 (&reg)[8]) {
        uint32_t kb = (uint32_t)kt * 128u;
        // a chunk wholly past K reads the (in-row) chunk holding element K - 1 instead
        if (!chunk_in(kt)) kb = (uint32_t)(((K - 1) / kPer) * kPer * kEsz) - (tid & 7) * 16;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          reg[i] = *reinterpret_cast<const u32x4 *>(bp[i] + (uint32_t)(off[i] + kb));
      };
      auto store_rows = [&](char *dst, const u32x4 (&reg)[8], int kt) {
        const bool z = !chunk_in(kt);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4 *>(dst + (r_base + 32 * i) * kRowBytes + (tid & 7) * 16) =
              z ? u32x4{0u, 0u, 0u, 0u} : reg[i];
      };
      u32x4 ra[8], rb[8];
      auto load_stage = [&](int kt) {
        load_rows(a_bp, a_off, kt, ra);
        load_rows(b_bp, b_off, kt, rb);
      };
      auto store_stage = [&](int st, int kt) {
        char *As = smem + st * 2 * kOpBytes;
        store_rows(As, ra, kt);
        store_rows(As + kOpBytes, rb, kt);
      };
      const int frag_row = lane & 15;
      const int a_frag = (wm * 128 + frag_row) * kRowBytes + (lane >> 4) * 16;
      const int b_frag = (wn * 128 + frag_row) * kRowBytes + (lane >> 4) * 16;
      load_stage(0);
      store_stage(0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) load_stage(kt + 1);
        const char *As = smem + st * 2 * kOpBytes;
        const char *Bs = As + kOpBytes;
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // the stage row's two 64-byte K slices
          u32x4 fa[8], fb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            fa[i] = *reinterpret_cast<const u32x4 *>(As + a_frag + i * 16 * kRowBytes + q * 64);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            fb[j] = *reinterpret_cast<const u32x4 *>(Bs + b_frag + j * 16 * kRowBytes + q * 64);
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
        }
        if (kt + 1 < nk) store_stage(st ^ 1, kt + 1);
        __syncthreads();
      }
    } else {
      // ============ bf16: LDS-direct loads, double-buffered 64-element K stages ============
      // A stage holds 64 K elements (128 bytes) of each of the 256 tile rows of both
      // operands, [256 rows][8 chunks of 16 B] per operand; logical chunk c of row r
      // sits at position c ^ ((r >> 1) & 7), so the 16 rows that a fragment read
      // touches together fall on distinct banks.  A load instruction fetches whole
      // 128-byte row segments (8 lanes per row), which the cache serves with one
      // request per row -- half the requests of 64-byte segments.  Loads go straight
      // from global memory into LDS (lane l writes 16 bytes at the instruction's LDS
      // base + 16 l), no VGPRs stage the data; stage kt+1 streams into the other
      // buffer while stage kt is multiplied.
      constexpr int kBKv = 128 / (int)sizeof(T);  // K elements per stage: 64 bf16 or 128 fp8
      const int nkv = (int)cdiv(K, kBKv);
      const bool ktail = (K % kBKv) != 0;
      auto swz = [](int r) { return (r >> 1) & 7; };
      auto rsrc = [](const char *base, int64_t bytes) {
        const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, (int)n, 0x00020000);
      };
      // Wave w loads tile rows [64 w, 64 w + 64), segments 2w and 2w+1 of the operand; its
      // load instruction k (0..7) covers rows 64 w + 8 k .. + 7, of segment 2w + k / 4.
      auto load_row = [&](int k) { return 64 * wave + 8 * k + (lane >> 3); };
      auto load_chunk = [&](int k) { return (lane & 7) ^ swz(load_row(k)); };
      // A wave's two segments are contiguous in memory for every operand except the
      // hidden-gradient staging rows (span pieces), so only that one takes a descriptor
      // per segment; the others take one per wave (scalar registers are at their limit).
      constexpr bool kSplitA = KIND == kDhidden;
      // (separate variables: the host compiler rejects arrays of the descriptor type)
      __amdgpu_buffer_rsrc_t ra0, ra1, rb;
      uint32_t a_vo[8], b_vo[8];  // per load instruction: this lane's byte offset at k = 0
      auto setup = [&](auto split, const RowSrc &s, __amdgpu_buffer_rsrc_t &r0, __amdgpu_buffer_rsrc_t &r1,
                       uint32_t (&vo)[8]) {
        constexpr bool kSplit = decltype(split)::value;
        const char *b0, *b1;
        int64_t n0, n1;
        seg<kSplit>(s, 2 * wave, b0, n0);
        seg<kSplit>(s, 2 * wave + 1, b1, n1);
        if (kSplit) {
          r0 = rsrc(uni(b0), uni(n0 * s.ldb));
          r1 = rsrc(uni(b1), uni(n1 * s.ldb));
        } else {
          r0 = rsrc(uni(b0), uni((n0 + n1) * s.ldb));
          r1 = r0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          vo[k] = (uint32_t)((int64_t)(load_row(k) & (kSplit ? 31 : 63)) * s.ldb) + (uint32_t)(load_chunk(k) * 16);
      };
      setup(std::integral_constant<bool, kSplitA>{}, srcA, ra0, ra1, a_vo);
      setup(std::false_type{}, srcB, rb, rb, b_vo);
      // LDS offset of operand op (0 = A, 1 = B) of stage s: bf16 [A0 B0 | A1 B1]; fp8
      // [A0 A1 | B0 B1], so that each operand's two stages lie within one 16-bit ds_read
      // offset of a per-lane base (the fp8 loop then reads with no address arithmetic)
      auto stage_op = [](int s, int op) -> int {
        return kF8 ? op * 2 * kOpStage + (s & 1) * kOpStage : (s & 1) * kStage + op * kOpStage;
      };
      // load k (0..7) of operand op (0 = A, 1 = B) of stage s
      auto issue_one = [&](int s, int op, int k) {
        char *lb = smem + stage_op(s, op) + (8 * wave + k) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rb : (kSplitA && k >= 4 ? ra1 : ra0), lb, 16,
                                                 op ? b_vo[k] : a_vo[k], s * 128, 0, 0);
      };
      // L2 prefetch.  The 32 workgroups of an XCD hold a kGroupM x (32 / kGroupM) block of
      // tiles and share operand rows through its L2; a line a stage needs that no sharer
      // has fetched yet misses, and every sharer then waits for that miss.  So each
      // workgroup touches, kPfAhead stages early, a share of the block's lines: of its A
      // tile's eight 32-row segments segment 2 (n % 4) + w for wave w = 0, 1, of its B
      // tile's segment m % 8 (waves 2 and 3), where (m, n) is its tile; one 128-byte line
      // per row per stage (two lanes, one per 64-byte half), with 4-byte loads into a
      // scratch corner of LDS: for the 8 x 4 block, each line once.  The load
      // goes out after the stage's real loads, so the wait for those can leave it in
      // flight (vector loads complete in order).
      // Measured per kind at two stages ahead: without it d-logits is 7% and dWeight 15%
      // slower; the forward gains about 1%.
      constexpr int kPfAhead = 2;  // 1 was as slow as none, 3 4-7% slower on dWeight
      constexpr bool kPrefetch = true;
      __amdgpu_buffer_rsrc_t rpf = rsrc(Wp, 0);
      uint32_t pf_vo = 0;
      if constexpr (kPrefetch) {
        const bool isA = wave < 2;
        // segment of 32 rows to touch, wave-uniform
        const int sg = isA ? 2 * (int)(ni & 3) + (wave & 1) : (int)(mi & 7);
        const char *pb_a, *pb_b;
        int64_t pn_a, pn_b;
        seg<kSplitA>(srcA, sg, pb_a, pn_a);
        seg<false>(srcB, sg, pb_b, pn_b);
        rpf = isA ? rsrc(uni(pb_a), uni(pn_a * srcA.ldb)) : rsrc(uni(pb_b), uni(pn_b * srcB.ldb));
        // lanes 0..31 touch the first 64 bytes of their row's line, lanes 32..63 the rest
        pf_vo = (uint32_t)((int64_t)(lane & 31) * (isA ? srcA.ldb : srcB.ldb)) + (uint32_t)((lane >> 5) * 64);
      }
      // Issued for every stage, so the vmcnt targets are constant; a stage past K touches
      // the last stage again (the scalar offset is not range-checked, so it must stay
      // inside the rows).
      auto issue_pf = [&](int s) {
        if constexpr (kPrefetch)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rpf, smem + kPfLds + wave * 256, 4, pf_vo,
                                                   (s < nkv ? s : nkv - 1) * 128, 0, 0);
      };
      // Last, partial K stage: chunks wholly past K were read from the next row (or
      // as zeros); overwrite them with zeros once this wave's loads of the stage have
      // landed.  A chunk that straddles K is kept: past K it holds the zero padding
      // of the token-major staging, of the split's block of W^T, of h^T or of the
      // vocabulary-major staging.
      auto fix_tail = [&](int s) {
        if (!(ktail && s == nkv - 1)) return;
        char *lb = smem + stage_op(s, 0);
        constexpr int kBOff = kF8 ? 2 * kOpStage : kOpStage;  // B relative to A of the same stage
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((int64_t)s * kBKv + load_chunk(k) * kPer >= K) {
            *reinterpret_cast<u32x4 *>(lb + (8 * wave + k) * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(lb + kBOff + (8 * wave + k) * 1024 + lane * 16) =
                u32x4{0u, 0u, 0u, 0u};
          }
      };
      constexpr int kVm0 = 0x0f70;    // s_waitcnt vmcnt(0) only (gfx9 encoding)
      constexpr int kVm1 = 0x0f71;    // vmcnt(1): all but the latest (prefetch) load
      constexpr int kLgkm0 = 0xc07f;  // s_waitcnt lgkmcnt(0) only
      constexpr int kVmNext = kPrefetch ? kVm1 : kVm0;  // a stage's own loads landed

      const int swz_lane = swz(lane & 15);  // same for every fragment row of this lane
      if constexpr (kF8) {
        // ============ fp8 (OCP E4M3): one 16 x 16 x 128 MFMA K step per stage ============
        // A stage holds 128 K elements (128 bytes) per row, the bytes of a bf16 stage, and
        // one v_mfma_f32_16x16x128_f8f6f4 per (i, j) block consumes all of them: a
        // fragment is 16 rows x 128 bytes, lane l holding row l % 16 and the 32 bytes at
        // K byte 32 (l / 16), logical chunks 2 (l / 16) and 2 (l / 16) + 1.  A and B use
        // the same lane -> K map, so every K element meets itself.  The instruction's
        // format fields are left at 0: both operands E4M3.
        //
        // A stage's 64 MFMAs run in quadrant order: blocks i, j < 4 (MFMA p = 4 i + j), then
        // i < 4, j >= 4, then i >= 4, j < 4, then i, j >= 4.  So A0..A3 and B0..B3 are
        // needed from the stage's first MFMA, B4..B7 from MFMA 16 and A4..A7 from MFMA 32,
        // and the previous stage released A0..A3 after its MFMA 31, B0..B3 after 47 and
        // the rest at its end.  One set of 16 fragments (128 VGPRs) then suffices: B4..B7
        // and A4..A7 of a stage are read during its first 32 MFMAs, one fragment beside
        // every fourth; the barrier before MFMA kBar8 publishes the next stage, whose
        // A0..A3 and B0..B3 are read right after it, one beside every second MFMA, into
        // registers this stage no longer needs.  All reads of a stage fall between the
        // barrier that publishes it and the next one, so after that next barrier its
        // buffer can take the loads of the stage after next.
        //
        // Loads, one beside every third MFMA: the B loads of stage kt + 1 early in stage
        // kt (before its barrier), the A loads of stage kt + 2 after it.
        typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
        typedef int i32x8 __attribute__((ext_vector_type(8)));
        // Schedule (MFMA indices p of a stage): this stage's B4..B7, A4..A7 read beside
        // p = kCurRd8 * f (f = 0..7); B loads of the next stage beside p = kB0_8 + kLoad8 m;
        // the L2 prefetch at kPf8At; the barrier before p = kBar8; the next stage's A0..A3
        // read beside kBar8 + 2 f, its B0..B3 beside kNxB8 + 2 f (B_j is last used at
        // p = 44 + j); A loads of the stage after next beside kBar8 + 1 + kLoad8 m.
        constexpr int kBar8 = 40, kLoad8 = 3, kB0_8 = 1, kCurRd8 = 4, kPf8At = 24;
        constexpr int kNxB8 = kBar8 + 8 > 48 ? kBar8 + 8 : 48;
        static_assert(4 * kCurRd8 <= 16 && 7 * kCurRd8 < kBar8, "B4.. read by MFMA 16, A7 before the barrier");
        static_assert(kB0_8 + 7 * kLoad8 < kPf8At && kPf8At < kBar8, "B loads, then the prefetch, before the barrier");
        static_assert(kBar8 + 1 + 7 * kLoad8 <= 63 && kNxB8 + 6 <= 63, "the stage's tail holds its loads and reads");
        // This lane's byte offsets of its two chunks in row (lane % 16) of block 0 of each
        // operand's buffer-0 stage; block blk of a stage in buffer b is at these plus
        // b * kOpStage + 2048 blk.  Each stage adds its buffer's term once, at its start
        // (`FragBase`, pinned in registers), so that a fragment read takes no address
        // arithmetic: every fragment register stays live until the read that replaces it
        // (see keep below), and an address computed between the two could otherwise land
        // in registers an 8-pass MFMA is still reading.
        int ro[2][2];
        {
          const int c0 = 2 * (lane >> 4);
#pragma unroll
          for (int op = 0; op < 2; ++op)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              ro[op][hh] = stage_op(0, op) + ((op ? wn : wm) * 128 + (lane & 15)) * 128 + (((c0 + hh) ^ swz_lane) << 4);
        }
        struct FragBase {
          int o[2][2];
        };
        auto frag_base = [&](int st) -> FragBase {
          FragBase b;
#pragma unroll
          for (int op = 0; op < 2; ++op)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              b.o[op][hh] = ro[op][hh] + (st & 1) * kOpStage;
              asm volatile("" : "+v"(b.o[op][hh]));  // computed here, not next to a read
            }
          return b;
        };
        auto read_frag8 = [&](const FragBase &b, int op, int blk) -> u32x8 {
          const char *lb = smem + 2048 * blk;
          const u32x4 lo = *reinterpret_cast<const u32x4 *>(lb + b.o[op][0]);
          const u32x4 hi = *reinterpret_cast<const u32x4 *>(lb + b.o[op][1]);
          return u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        };
        u32x8 fa[8], fb[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) fa[f] = fb[f] = u32x8{0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        // A fragment's registers stay allocated to it until the read that replaces it: the
        // compiler sees the inline MFMA's operands as consumed once it is issued and would
        // otherwise reuse them for addresses while the 8-pass instruction still reads them.
        auto keep = [](const u32x8 &x) { asm volatile("" : : "v"(x)); };
        // `last`: the tile's last stage, with the compiler's MFMA (it then owns the wait
        // states of the epilogue that reads the accumulators)
        auto mma8 = [&](bool last, int i, int j) {
          if (last)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                __builtin_bit_cast(i32x8, fa[i]), __builtin_bit_cast(i32x8, fb[j]), acc[i][j], 0, 0, 0, 0, 0, 0);
          else
            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fa[i]), "v"(fb[j]));
        };
        auto kstep8 = [&](int kt, bool last) {
          const FragBase bc = frag_base(kt), bn = frag_base(kt + 1);
#pragma unroll
          for (int p = 0; p < 64; ++p) {
            if (p % kCurRd8 == 0 && p / kCurRd8 < 8) {  // this stage's B4..B7, then A4..A7
              const int f = p / kCurRd8;
              if (f < 4) {
                keep(fb[4 + f]);
                fb[4 + f] = read_frag8(bc, 1, 4 + f);
              } else {
                keep(fa[f]);
                fa[f] = read_frag8(bc, 0, f);
              }
            }
            if (!last && p >= kB0_8 && (p - kB0_8) % kLoad8 == 0 && (p - kB0_8) / kLoad8 < 8)
              issue_one(kt + 1, 1, (p - kB0_8) / kLoad8);  // B loads of kt + 1
            if (!last && p == kPf8At) issue_pf(kt + 1 + kPfAhead);
            if (!last && p == kBar8) {
              __builtin_amdgcn_s_waitcnt(kVmNext);  // this wave's loads of stage kt + 1 have landed
              fix_tail(kt + 1);
              __builtin_amdgcn_s_waitcnt(kLgkm0);  // and its reads of stage kt are done
              __builtin_amdgcn_s_barrier();
            }
            if (!last && p >= kBar8 && p < kBar8 + 8 && ((p - kBar8) & 1) == 0) {  // next stage's A0..A3
              const int f = (p - kBar8) >> 1;
              keep(fa[f]);
              fa[f] = read_frag8(bn, 0, f);
            }
            if (!last && p >= kNxB8 && p < kNxB8 + 8 && ((p - kNxB8) & 1) == 0) {  // and B0..B3
              const int f = (p - kNxB8) >> 1;
              keep(fb[f]);
              fb[f] = read_frag8(bn, 1, f);
            }
            if (p > kBar8 && (p - kBar8 - 1) % kLoad8 == 0 && (p - kBar8 - 1) / kLoad8 < 8 && kt + 2 < nkv)
              issue_one(kt + 2, 0, (p - kBar8 - 1) / kLoad8);  // A loads of kt + 2
            const int q = p >> 4, r = p & 15;
            mma8(last, ((q & 2) ? 4 : 0) + (r >> 2), ((q & 1) ? 4 : 0) + (r & 3));
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        // The zeroed accumulators are pinned here, long before the first inline MFMA that
        // accumulates into them (left alone, the compiler sinks each zeroing to just before
        // that MFMA, closer than the matrix core's operand wait states allow).
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) asm volatile("" : "+a"(acc[i][j]));
        // ---- prologue: stage 0 loaded and visible, its A0..A3 and B0..B3 read, the A
        // loads of stage 1 issued ----
#pragma unroll
        for (int k8 = 0; k8 < 16; ++k8) issue_one(0, k8 >> 3, k8 & 7);
        __builtin_amdgcn_s_waitcnt(kVm0);
        fix_tail(0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        {
          const FragBase b0 = frag_base(0);
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            fa[f] = read_frag8(b0, 0, f);
            fb[f] = read_frag8(b0, 1, f);
          }
        }
        if (nkv > 1) {
#pragma unroll
          for (int k = 0; k < 8; ++k) issue_one(1, 0, k);
        }
        __builtin_amdgcn_sched_barrier(0);
        for (int kt = 0; kt + 1 < nkv; ++kt) kstep8(kt, false);
        kstep8(nkv - 1, true);
      } else {
      // Fragment of block i (16 rows from wbase + 16 i) for K slice q (0, 1: 32 elements,
      // 64 bytes) of a stage: lane l reads row l % 16, logical chunk 4 q + l / 16.
      auto read_frag = [&](const char *op, int wbase, int i, int q) -> u32x4 {
        const int R = wbase + 16 * i + (lane & 15);
        return *reinterpret_cast<const u32x4 *>(op + R * 128 + (((4 * q + (lane >> 4)) ^ swz_lane) << 4));
      };
      // Fragment read p (0..15) of K slice q of stage s, in the order the MFMAs consume
      // them: A0, B0..B7, A1..A7.
      auto read_one = [&](int s, int q, int p, u32x4 (&fa)[8], u32x4 (&fb)[8]) {
        const char *lb = smem + (s & 1) * kStage;
        if (p == 0)
          fa[0] = read_frag(lb, wm * 128, 0, q);
        else if (p < 9)
          fb[p - 1] = read_frag(lb + kOpStage, wn * 128, p - 1, q);
        else
          fa[p - 8] = read_frag(lb, wm * 128, p - 8, q);
      };
      // A stage is two K steps of 64 MFMAs, (i, j) = (p / 8, p % 8) for MFMA p.  A
      // scheduling fence after every MFMA keeps the order written here.
      //
      // Right after the barrier that publishes a stage every wave reads at once, so the
      // LDS is busiest there.  Only the first kPostReads fragments of the stage's slice 0
      // (A0, B0..B7, A1) are read then; A2..A7 follow in the first step, fragment A(i)
      // beside MFMA 8 (i - 2), a row of 8 MFMAs before its row starts.
      constexpr int kPostReads = 10;
      static_assert(kPostReads >= 10 && kPostReads <= 16, "A(i), i >= 2, are read in the first step");
      auto read_slice0_a = [&](int s, int p, u32x4 (&fa)[8]) {  // read p (>= 9) of slice 0 = A(p - 8)
        fa[p - 8] = read_frag(smem + (s & 1) * kStage, wm * 128, p - 8, 0);
      };
      //
      // First step (fragments ca, cb): beside MFMA 2k + 1 (k < 16) fragment read k of
      // slice 1 of this stage into (na, nb); beside MFMA kLoadEvery * k + 1, load k of stage
      // ls (if ls >= 0; A then B); after the last load, the L2 prefetch of stage pfs;
      // beside MFMA 8 m, the read of A(m + 2) of slice 0 into ca unless it was read after
      // the barrier.
      //
      // The loads are spread over the step because the path from L2 into LDS is the
      // narrow part: a probe measured about 55 bytes per clock per CU into LDS at best,
      // and a stage is 64 KiB per workgroup, so 16 loads per wave within 32 MFMAs (512
      // clocks) arrive at over twice that rate and queue, while every load still hitting
      // L2 leaves the loop almost as slow as it is.  Loads later in the step have less time
      // to land before the barrier that publishes their stage.
      constexpr int kLoadEvery = 4;  // 2: 3% slower per step; 3: 0.4% slower
      static_assert(15 * kLoadEvery + 1 < 64, "a stage's loads are issued in its first step");
      constexpr int kPfAt = 16 * kLoadEvery < 64 ? 16 * kLoadEvery : 63;
      static_assert(kPfAt > 15 * kLoadEvery + 1, "the prefetch goes out after the stage's last load");
      // `last`: the tile's last stage, with the compiler's MFMA (see Mma).
      auto mma = [&](bool last, int p, const u32x4 (&ca)[8], const u32x4 (&cb)[8]) {
        if (last)
          Mma<T>::run(acc[p >> 3][p & 7], ca[p >> 3], cb[p & 7]);
        else
          Mma<T>::run_in_place(acc[p >> 3][p & 7], ca[p >> 3], cb[p & 7]);
      };
      auto kstep0 = [&](u32x4 (&ca)[8], const u32x4 (&cb)[8], u32x4 (&na)[8], u32x4 (&nb)[8],
                        int rs, int ls, int pfs, bool last) {
#pragma unroll
        for (int p = 0; p < 64; ++p) {
          if ((p & 7) == 0 && 10 + (p >> 3) >= kPostReads && 10 + (p >> 3) < 16)
            read_slice0_a(rs, 10 + (p >> 3), ca);
          if (p < 32 && (p & 1)) read_one(rs, 1, p >> 1, na, nb);
          if (ls >= 0 && p % kLoadEvery == 1 && p / kLoadEvery < 16)
            issue_one(ls, (p / kLoadEvery) >> 3, (p / kLoadEvery) & 7);
          if (pfs >= 0 && p == kPfAt) issue_pf(pfs);
          mma(last, p, ca, cb);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // Second step: kBarAt MFMAs; then, if there is a next stage, wait for its loads,
      // publish it (barrier) and read the first kPostReads fragments of its slice 0 into
      // (na, nb), one beside each of the remaining MFMAs.
      constexpr int kBarAt = 52;
      static_assert(64 - kBarAt >= kPostReads, "one read per MFMA after the barrier");
      auto kstep1 = [&](const u32x4 (&ca)[8], const u32x4 (&cb)[8], u32x4 (&na)[8], u32x4 (&nb)[8],
                        bool next, int ns) {
#pragma unroll
        for (int p = 0; p < kBarAt; ++p) {
          mma(!next, p, ca, cb);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (next) {
          __builtin_amdgcn_s_waitcnt(kVmNext);  // this wave's loads of stage ns have landed
          fix_tail(ns);
          __builtin_amdgcn_s_waitcnt(kLgkm0);  // and its reads of this stage are done
          __builtin_amdgcn_s_barrier();
        }
#pragma unroll
        for (int p = kBarAt; p < 64; ++p) {
          if (next && p - kBarAt < kPostReads) read_one(ns, 0, p - kBarAt, na, nb);
          mma(!next, p, ca, cb);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // ---- prologue: stage 0 loaded and visible, its slice 0 read ----
#pragma unroll
      for (int k8 = 0; k8 < 16; ++k8) issue_one(0, k8 >> 3, k8 & 7);
      __builtin_amdgcn_s_waitcnt(kVm0);
      fix_tail(0);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      u32x4 F0a[8], F0b[8], F1a[8], F1b[8];
#pragma unroll
      for (int p = 0; p < kPostReads; ++p) read_one(0, 0, p, F0a, F0b);
      __builtin_amdgcn_sched_barrier(0);

      // Stage kt: stage kt+1 streams into the other buffer (which held stage kt-1,
      // released by the previous barrier) during the first step; the second step
      // publishes it.  The last stage is peeled so the loop body is one straight path.
      for (int kt = 0; kt + 1 < nkv; ++kt) {
        kstep0(F0a, F0b, F1a, F1b, kt, kt + 1, kt + kPfAhead, false);
        kstep1(F1a, F1b, F0a, F0b, true, kt + 1);
      }
      kstep0(F0a, F0b, F1a, F1b, nkv - 1, -1, -1, true);
      kstep1(F1a, F1b, F0a, F0b, false, 0);
      }  // bf16 schedule
      __builtin_amdgcn_s_waitcnt(kVm0);  // prefetches still in flight target LDS
      __syncthreads();  // every wave is done with the ring before epilogues reuse LDS
    }

    // ---------------- epilogues ----------------
    // acc[i][j][x] holds tile row  wm*128 + i*16 + 4*(lane / 16) + x
    //               and tile col  wn*128 + j*16 + (lane % 16).
    // Indices below are tile-local 32-bit; tile origins are uniform.
    // Epilogue addresses depend only on the lane; computed from an opaque copy of the
    // lane index here, they cannot be hoisted out of the tile loop and held in
    // registers through the main loop.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const int row0 = wm * 128 + ((elane >> 4) << 2);  // + i*16 + x
    const int col0 = wn * 128 + (elane & 15);         // + j*16
    // bf16 epilogues stage a 256 x 256 bf16 tile in LDS column-major, Ls[col][row] with
    // kLsPitch-byte lines (a lane's 4 consecutive rows are one 8-byte write), and write
    // it out row by row with transposing LDS reads: in a group of 16 lanes, lane i
    // names 4 consecutive rows (mb + 4 (i % 4)) of column line cb + i / 4 and receives
    // row mb + i over columns cb .. cb + 3; two reads give 8 columns, one 16-byte store.
    // A wave store writes 64 contiguous bytes of each of 16 rows.  Row m (< m_valid)
    // goes to dst + m * ld elements (streaming stores if kNt); colmap(cb) gives the
    // destination column of tile columns cb .. cb + 7, or -1 to skip them.
    auto ls_put4 = [&](int col, int c0, float d0, float d1, float d2, float d3) {
      u32x2 v;
      v.x = bf16x2_rne(d0, d1);
      v.y = bf16x2_rne(d2, d3);
      *reinterpret_cast<u32x2 *>(smem + col * kLsPitch + c0 * 2) = v;
    };
    auto ls_store_rows = [&](auto nt, char *dst, int64_t ld, int m_valid, auto &&colmap) {
      constexpr bool kNt = decltype(nt)::value;
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      const int li = elane & 15, g4 = elane >> 4;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        const int mb = wave * 64 + vb * 16;
#pragma unroll 2
        for (int k = 0; k < 8; ++k) {
          const int cb = k * 32 + g4 * 8;  // first of this lane's 8 columns
          const char *src = smem + (cb + (li >> 2)) * kLsPitch + (mb + 4 * (li & 3)) * 2;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(src));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (s16x4 __attribute__((address_space(3))) *)(src + 4 * kLsPitch));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const int64_t c = colmap(k, cb);
          if (c >= 0 && mb + li < m_valid) {
            char *p = dst + ((int64_t)(mb + li) * ld + c) * 2;
            if constexpr (kNt)
              store16_nt(p, u32x4{l2.x, l2.y, h2.x, h2.y});
            else
              *reinterpret_cast<u32x4 *>(p) = u32x4{l2.x, l2.y, h2.x, h2.y};
          }
        }
      }
    };
    if constexpr (KIND == kFwd || KIND == kFwdSkip) {
      // Per token (column) of the tile: max M of its logits over the tile's vocabulary
      // rows, s = sum e^(z - M), u = sum e^(z - M) (z - M).  Exponentials are taken in
      // base 2 (d = (z - M) log2 e, e = 2^d, u = ln 2 * sum e d); each sum runs as four
      // independent chains (row blocks i and i + 4), since a single wave per SIMD cannot
      // hide a long dependent chain.  The target's logit is not picked out here: it is
      // one dot product per token, taken beside the merge of the tile states.
      const int64_t v_tile = mi * kTile;
      const int n_rows = (int)imin(a.V - v_tile, kTile);  // valid vocabulary rows
      const int64_t t_tile = ni * kTile;
      constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
      // Rows past the vocabulary (last tile only) read as a large finite negative logit:
      // its exponential is 0 and 0 * d stays 0.  A wave with no valid row at all
      // reports the empty state instead.  The masked and the plain epilogue are two
      // instances of one body, so the accumulators are only ever read.
      const bool wave_live = wm * 128 < n_rows;
      const int row_lim = n_rows - row0;  // tile row row0 + off is valid iff off < row_lim
      float4 *xch = reinterpret_cast<float4 *>(smem);
      float st_M[8], st_s[8], st_u[8];
      // The logits are the accumulators times zscale (1 for bf16 and fp32 inputs; for
      // fp8 inputs the product of the two tensors' scales, > 0, so the maximum of the
      // scaled values is the scaled maximum).
      const float zs = kF8 ? a.zscale : 1.f;
      const float zl2 = zs * kLog2e;
      auto softmax_states = [&](auto masked) {
        constexpr bool kMasked = decltype(masked)::value;
        // an invalid row (past the vocabulary) reads as a large negative accumulator: it
        // never wins the maximum and its exponential is 0 (fp8: the scaled value may reach
        // -inf, so the exponent is clamped below, where 2^d is 0 and 0 * d adds nothing)
        auto z_at = [&](int i, int j, int x) -> float {
          const float z = acc[i][j][x];
          if constexpr (kMasked)
            return i * 16 + x < row_lim ? z : (kF8 ? -3.0e38f : -1.0e30f);
          else
            return z;
        };
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // chain c takes row blocks c and c + 4
          float m4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            m4[c] = z_at(c, j, 0);
#pragma unroll
            for (int e = 1; e < 8; ++e) m4[c] = fmaxf(m4[c], z_at(c + 4 * (e >> 2), j, e & 3));
          }
          float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
          mx = max_over_x16_x32(mx) * zs;  // the column's 4 lane groups; scaled
          const float nm2 = -mx * kLog2e;
          float s4[4], u4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            s4[c] = 0.f;
            u4[c] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float d = __builtin_fmaf(z_at(c + 4 * (e >> 2), j, e & 3), zl2, nm2);
              if constexpr (kF8 && kMasked) d = fmaxf(d, -1000.f);
              const float ex = __builtin_amdgcn_exp2f(d);
              s4[c] += ex;
              u4[c] = __builtin_fmaf(ex, d, u4[c]);
            }
          }
          float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
          float u = (u4[0] + u4[1]) + (u4[2] + u4[3]);
          s = sum_over_x16_x32(s);
          u = sum_over_x16_x32(u);
          u *= kLn2;
          if (!wave_live) {
            mx = kNegInf;
            s = 0.f;
            u = 0.f;
          }
          st_M[j] = mx;
          st_s[j] = s;
          st_u[j] = u;
          if (wm == 1 && elane < 16) xch[col0 + j * 16] = make_float4(mx, s, u, 0.f);
        }
      };
      if (n_rows < kTile)
        softmax_states(std::true_type{});
      else
        softmax_states(std::false_type{});
      __syncthreads();
      if (wm == 0 && elane < 16) {
        // tokens of the tile's columns: t_tile + col, or (pairs of active tiles) the
        // first token of this wave's tile (columns wn * 128 ..) + col % 128
        int64_t t_first = t_tile;
        int n_cols = (int)imin(a.T - t_tile, kTile);
        if constexpr (KIND == kFwdSkip) {
          const int64_t tile = uni(2 * ni + wn < uni(a.counts[0]) ? a.tile_list[2 * ni + wn] : -1);
          t_first = tile < 0 ? 0 : tile * kSkipTile - wn * 128;
          n_cols = tile < 0 ? 0 : (int)imin(a.T - tile * kSkipTile + wn * 128, kTile);
        }
        float4 *out = reinterpret_cast<float4 *>(a.part) + mi * a.T + t_first;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = col0 + j * 16;
          const float4 o = xch[col];
          float M = st_M[j], s = st_s[j], u = st_u[j];
          merge_state(M, s, u, o.x, o.y, o.z);
          if (col < n_cols) out[col] = make_float4(M, s, u, 0.f);
        }
      }
    } else if constexpr (KIND == kDlogits) {
      const int64_t v_tile = mi * kTile;  // split-local first column
      const int n_live = (int)imin(a.Ws - v_tile, kTile);
      const int n_cols = (int)imin(cdiv(a.Ws_grid, kSPer) * kSPer - v_tile, kTile);  // written columns
      const int64_t t_pad = cdiv(a.T, kSPer) * kSPer;  // tokens written, zero padding included
      // the pair's two token tiles (the second may be missing)
      const int64_t n_act = uni(a.counts[0]);  // active token tiles
      const int64_t pt0 = uni(a.tile_list[2 * ni]);
      const int64_t pt1 = (2 * ni + 1 < a.n_skip_tiles) ? uni(a.tile_list[2 * ni + 1]) : -1;
      TS *Dd = reinterpret_cast<TS *>(a.D) + v_tile;
      TS *Dv = reinterpret_cast<TS *>(a.Dt) + v_tile * a.ld_t;
      // bf16: the tile's d-logits are staged in LDS token-major, Ls[token][vocab] with
      // kLsPitch-byte rows, and both layouts are then written with 16-byte stores.
      char *Ls = smem;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = col0 + j * 16;               // token within the pair tile
        const int64_t tile = wn ? pt1 : pt0;         // col / 128 == wn
        const int64_t t = tile * kSkipTile + (col & 127);
        const bool tok = tile >= 0 && t < a.T;
        bool act = false;
        float lse_t = 0.f, ez = 0.f, ga = 0.f, gb = 0.f;
        int yl = -1;
        if (tok) {
          act = a.mask ? (a.mask[t] != 0) : true;
          if (act) {
            lse_t = a.lse[t];
            ez = lse_t - a.entropy[t];
            ga = a.grad_lp ? a.grad_lp[t] : 0.f;
            gb = a.grad_ent ? a.grad_ent[t] : 0.f;
            const int64_t yd = a.targets[t] - a.v_base - v_tile;
            yl = (yd >= 0 && yd < kTile) ? (int)yd : -1;
          }
        }
        const int lim = act ? n_live : 0;  // columns >= lim are 0
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c0 = row0 + i * 16;  // first of 4 consecutive vocabulary rows
            float d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float z = kF8 ? acc[i][j][c] * a.zscale : acc[i][j][c];  // fp8: codes' product x scales
              const float p = __expf(z - lse_t);
              const float val = ga * ((c0 + c == yl ? 1.f : 0.f) - p) + gb * p * (ez - z);
              d[c] = (c0 + c < lim) ? val : 0.f;
            }
            if constexpr (kV2) {
              ls_put4(col, c0, d[0], d[1], d[2], d[3]);
            } else {
              if (tok && c0 < n_cols) store4(Dd + t * a.ld_d + c0, d[0], d[1], d[2], d[3]);
              // vocabulary-major column: the token, or its slot among the active tiles
              const int64_t rank = 2 * ni + (col >> 7);
              const int64_t tc = a.compact_dw ? rank * kSkipTile + (col & 127) : t;
              if (tile >= 0 && (a.compact_dw ? rank < n_act : t < t_pad)) {  // a token or padding
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (c0 + c < n_live) store1(Dv + (int64_t)(c0 + c) * a.ld_t + tc, d[c]);
              }
            }
          }
      }
      if constexpr (kV2) {
        __syncthreads();
        char *Db = reinterpret_cast<char *>(Dd);
        char *Dvb = reinterpret_cast<char *>(Dv);
        // token-major: row t, vocabulary columns [0, n_cols); each wave covers two
        // 512-byte rows per store
#pragma unroll 4
        for (int k = 0; k < 32; ++k) {
          const int tl = wave * 64 + 2 * k + (elane >> 5);  // token within the pair tile
          const int cc = (elane & 31) * 8;                  // first column of the chunk
          const u32x4 v = *reinterpret_cast<const u32x4 *>(Ls + tl * kLsPitch + cc * 2);
          const int64_t tile = (tl >> 7) ? pt1 : pt0;
          const int64_t t = tile * kSkipTile + (tl & 127);
          if (tile >= 0 && t < a.T && cc < n_cols)
            store16_nt(Db + (t * a.ld_d + cc) * 2, v);
        }
        // vocabulary-major: rows v of the split, tokens of the pair (zero padding to a
        // whole 16-byte chunk included)
        // first column of each of the pair's tiles: its first token, or (compact) its
        // slot among the active tiles; -1: not stored
        const bool cpt = a.compact_dw != 0;
        const int64_t vcol0 = uni(pt0 < 0 ? -1 : (cpt ? (2 * ni < n_act ? 2 * ni * kSkipTile : -1) : pt0 * kSkipTile));
        const int64_t vcol1 =
            uni(pt1 < 0 ? -1 : (cpt ? (2 * ni + 1 < n_act ? (2 * ni + 1) * kSkipTile : -1) : pt1 * kSkipTile));
        const int64_t vlim = uni(cpt ? a.ld_t : t_pad);
        ls_store_rows(std::true_type{}, Dvb, a.ld_t, n_live, [&](int k, int cb) -> int64_t {
          const int64_t base = (k >> 2) ? vcol1 : vcol0;  // cb / 128
          const int64_t c = base + (cb & 127);
          return (base >= 0 && c < vlim) ? c : -1;
        });
      }
    } else if constexpr (KIND == kDhidden) {
      const int64_t n_tile = ni * kTile;
      const int n_cols = (int)imin(a.H - n_tile, kTile);
      float *base = a.dh_acc + n_tile;  // + token * H
      if constexpr (kV2) {
        // fp32 sum over splits through LDS, half a tile at a time: in phase p every wave
        // writes its row blocks i = 4p .. 4p + 3 as they sit in registers,
        // [wave][i - 4p][j][x][lane] with 64 bytes of padding after each (i, j) group
        // (constant offsets from one per-lane base); then wave w takes the 32 rows of piece
        // 4 (w / 2) + 2p + w % 2 (tile rows (w / 2) * 128 + 64 p + 32 (w % 2) ..) and adds
        // the earlier splits' sum with 16-byte loads and stores (4 consecutive columns
        // are 4 consecutive lanes of one register).  The skew puts the 16 lanes of a
        // read on distinct banks.
        const int c4 = elane * 4;  // this lane's 4 columns in the row it handles
        // column c4 sits in the registers of wave (wm, wn = c4 / 128), j = c4 / 16 % 8,
        // lanes c4 % 16 + 16 g4 ..
        const int lds_col = (c4 >> 7) * kDhWave + ((c4 >> 4) & 7) * kDhGroup + (c4 & 15) * 4;
        char *wb = smem + wave * kDhWave + elane * 4;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int x = 0; x < 4; ++x)
                *reinterpret_cast<float *>(wb + (ii * 8 + j) * kDhGroup + x * 256) = acc[4 * p + ii][j][x];
          __syncthreads();
          const int rwm = wave >> 1, rh = wave & 1;  // the 32 rows this wave stores
          const int src_b = lds_col + rwm * 2 * kDhWave;  // + the row's (ii, g4, x)
          // the 32 rows are one span piece: tokens pst .., valid below pln
          int64_t pst, pln;
          piece(a.span_tiles, 8 * mi + 4 * rwm + 2 * p + rh, uni(a.counts[2]), pst, pln);
          const int n_in = (int)pln;
          float *bblk = base + pst * a.H;
#pragma unroll
          for (int k0 = 0; k0 < 32; k0 += 8) {
            float4 prev[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              const int rr = k0 + kk;
              const bool ok = !a.first_split && rr < n_in && c4 < n_cols;
              prev[kk] = ok ? *reinterpret_cast<const float4 *>(bblk + (uint32_t)rr * (uint32_t)a.H + c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
              // row rr of the piece: block ii = 2 rh + rr / 16, g4 = rr % 16 / 4, x = rr % 4
              const int rr = k0 + kk;
              const int src = src_b + 64 * ((rr & 15) >> 2) + (2 * rh + (rr >> 4)) * 8 * kDhGroup + (rr & 3) * 256;
              if (rr < n_in && c4 < n_cols) {
                float4 v = *reinterpret_cast<const float4 *>(smem + src);
                v.x += prev[kk].x;
                v.y += prev[kk].y;
                v.z += prev[kk].z;
                v.w += prev[kk].w;
                *reinterpret_cast<float4 *>(bblk + (uint32_t)rr * (uint32_t)a.H + c4) = v;
              }
            }
          }
          __syncthreads();
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // tile rows wm * 128 + 16 i + .. are rows 16 (i % 2) + .. of piece 4 wm + i / 2
          int64_t pst, pln;
          piece(a.span_tiles, 8 * mi + 4 * wm + (i >> 1), uni(a.counts[2]), pst, pln);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int lr = 16 * (i & 1) + 4 * (elane >> 4) + x;
            if (lr >= pln) continue;
            float *prow = base + (pst + lr) * a.H;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int col = col0 + j * 16;
              if (col < n_cols) prow[col] = acc[i][j][x];
            }
          }
        }
      }
    } else {
      const int64_t v_tile = mi * kTile;
      const int n_rows = (int)imin(a.Ws - v_tile, kTile);
      const int64_t n_tile = ni * kTile;
      const int n_cols = (int)imin(a.H - n_tile, kTile);
      T *base = reinterpret_cast<T *>(a.dW) + (a.v_base + v_tile) * a.H + n_tile;
      if constexpr (kV2) {
        // kDweightS: h^T holds the widened fp8 codes of h, so dW = out_scale * (D^T h^T)
        const float os = KIND == kDweightS ? a.out_scale : 1.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            ls_put4(col0 + j * 16, row0 + i * 16, acc[i][j][0] * os, acc[i][j][1] * os, acc[i][j][2] * os,
                    acc[i][j][3] * os);
        __syncthreads();
        ls_store_rows(std::false_type{}, reinterpret_cast<char *>(base), a.H, n_rows,
                      [&](int, int cb) -> int64_t { return cb < n_cols ? cb : -1; });
      } else {
        const uint32_t ldw = (uint32_t)a.H;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int row = row0 + i * 16 + x;
            if (row >= n_rows) continue;
            T *prow = base + (uint32_t)row * ldw;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int col = col0 + j * 16;
              if (col < n_cols) store1(prow + col, acc[i][j][x]);
            }
          }
      }
    }
    __syncthreads();  // LDS is reused by the next tile's prologue
  }
}

template <typename T, int KIND>
hipError_t launch_kind(const GemmArgs &a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<T, KIND>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(GemmKind kind, const GemmArgs &a, int grid, hipStream_t st) {
  switch (kind) {
    case kFwd: return launch_kind<T, kFwd>(a, grid, st);
    case kDlogits: return launch_kind<T, kDlogits>(a, grid, st);
    case kDhidden: return launch_kind<T, kDhidden>(a, grid, st);
    case kDweight: return launch_kind<T, kDweight>(a, grid, st);
    case kFwdSkip: return launch_kind<T, kFwdSkip>(a, grid, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, GemmKind kind, const GemmArgs &a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 2) {  // fp8 operands: the contractions over H (the hidden- and weight-gradient
                     // products take bf16 operands and run as dtype 1)
    switch (kind) {
      case kFwd: return launch_kind<uint8_t, kFwd>(a, grid, st);
      case kFwdSkip: return launch_kind<uint8_t, kFwdSkip>(a, grid, st);
      case kDlogits: return launch_kind<uint8_t, kDlogits>(a, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (kind == kDweightS)
    return dtype == 1 ? launch_kind<uint16_t, kDweightS>(a, grid, st) : hipErrorInvalidValue;
  return dtype == 1 ? launch_t<uint16_t>(kind, a, grid, st) : launch_t<float>(kind, a, grid, st);
}

}  // namespace flh
