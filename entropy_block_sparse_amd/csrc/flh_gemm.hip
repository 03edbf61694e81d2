// The four contractions of the fused LM head on CDNA4 matrix cores (gfx950).
//
//   forward   z^T = W h^T per (256 vocab x 256 token) tile, K = H, with the online
//             log-softmax statistics reduced in the epilogue (fused linear
//             log-prob and entropy: SkyRL #2376 "What does this PR do?" and the
//             stack's "fuse LM-head entropy for RL" layer).
//   d-logits  the same product recomputed for one vocabulary split over pairs of
//             active 128-token tiles only, with the d-logits of log-prob and
//             entropy formed in the epilogue and stored to the split's
//             live-width staging buffer ("How it works": only active d-logits
//             tiles are processed; the final split allocates its live width).
//   dHidden   D[span rows, :] W_s, accumulated in fp32 across splits, over
//             span-local row tiles only (Gemini "Code Review": d_hidden +=
//             split_d_logits @ split_weight; "How it works": spans, no token
//             reordering).
//   dWeight   D^T h over all tokens, dense ("How it works": weight gradients stay
//             a dense contraction).
//
// One kernel template serves all four.  A workgroup of 4 waves owns a 256 x 256
// output tile; each wave a 128 x 128 quadrant as 4 x 4 blocks of 32 x 32 MFMA
// accumulators (v_mfma_f32_32x32x16_bf16, or four v_mfma_f32_32x32x2_f32 per
// 16-byte fragment for fp32).  K is staged 128 bytes per row at a time through
// two LDS buffers (144-byte padded rows), so each K step costs one barrier and
// the next step's global loads are in flight during the current step's MFMAs.
// Operands whose K index is contiguous in memory (h, W, the d-logits rows) are
// loaded as 16-byte row chunks; operands whose K index is the row index (W and
// the d-logits for dHidden/dWeight) are loaded as 8 x 8 (bf16) or 4 x 4 (fp32)
// element blocks and transposed in registers before the LDS store, so no
// transposed copy of W, h or the d-logits is ever written to HBM.
//
// Workgroups are persistent (grid = compute units) and walk a tile list whose
// order keeps the tiles of one XCD (workgroup id mod 8) in a compact 8 x 4 block
// so operand tiles are shared in that XCD's L2.
#include <hip/hip_runtime.h>

#include "flh_internal.h"

namespace flh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kRowBytes = 144;               // LDS tile row: 128 B of K + 16 B pad
constexpr int kOpBytes = kTile * kRowBytes;  // one operand tile, one stage
constexpr int kLdsBytes = 4 * kOpBytes;      // A and B, two stages (147456 B)
// bf16 path: a ring of kNS stages of 32 K elements (64 B per row) per operand.
constexpr int kNS = 4;
constexpr int kOpStage = kTile * 64;         // one operand, one stage: 16 KiB
constexpr int kStage = 2 * kOpStage;         // 32 KiB
constexpr int kLdsBytesV2 = kNS * kStage;    // 128 KiB
constexpr float kNegInf = -__builtin_huge_valf();

template <typename T> struct Elt;
template <> struct Elt<uint16_t> { static constexpr int kPer = 8; };  // bf16 bit patterns
template <> struct Elt<float> { static constexpr int kPer = 4; };

__device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- matrix-core step: acc += a * b for one 16-byte fragment per lane ---------------
// Lane l feeds row (l % 32) of A and column (l % 32) of B with the K elements of
// the 16-byte chunk at position (l / 32) of a 32-byte K slice; A and B use the
// same lane -> K assignment, so every K element is paired with itself.
template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
  static __device__ __forceinline__ void run(f32x16 &c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16 &c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// ---- in-register transposes of a block of 16-byte rows ----------------------------
// in[i] holds K row i (kPer elements along M); out[j] holds M element j as kPer
// consecutive K values.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8], uint16_t) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const bool hi = j & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo_row = in[2 * i][w];
      const uint32_t hi_row = in[2 * i + 1][w];
      out[j][i] = hi ? ((lo_row >> 16) | (hi_row & 0xffff0000u))
                     : ((lo_row & 0xffffu) | (hi_row << 16));
    }
  }
}
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8], float) {
  // two independent 4 x 4 blocks: in[0..3] -> out[0..3], in[4..7] -> out[4..7]
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * b + j][i] = in[4 * b + i][j];
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store4(uint16_t *p, float a, float b, float c, float d) {
  u32x2 v;
  v.x = bf16_rne(a) | (bf16_rne(b) << 16);
  v.y = bf16_rne(c) | (bf16_rne(d) << 16);
  *reinterpret_cast<u32x2 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store1(uint16_t *p, float a) { *p = (uint16_t)bf16_rne(a); }
__device__ __forceinline__ void store1(float *p, float a) { *p = a; }

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

template <typename T, int KIND>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    const GemmArgs a) {
  constexpr bool kV2 = sizeof(T) == 2;  // bf16: LDS-direct ring; fp32: register-staged
  __shared__ __attribute__((aligned(16))) char smem[kV2 ? kLdsBytesV2 : kLdsBytes];
  constexpr int kPer = Elt<T>::kPer;       // elements per 16-byte chunk
  constexpr int kBK = 128 / sizeof(T);     // K elements per stage
  constexpr bool kATr = (KIND == kDweight);
  constexpr bool kBTr = (KIND == kDhidden || KIND == kDweight);
  constexpr int64_t kEsz = sizeof(T);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int g = lane >> 5;

  // ---------------- extents of this launch ----------------
  int64_t m_tiles, n_tiles, K;
  int64_t n_pairs_gemm = 0, n_pairs_all = 0;
  if constexpr (KIND == kFwd) {
    m_tiles = cdiv(a.V, kTile);
    n_tiles = cdiv(a.T, kTile);
    K = a.H;
  } else if constexpr (KIND == kDlogits) {
    m_tiles = cdiv(a.ld_d, kTile);
    n_pairs_gemm = cdiv(a.counts[0], 2);
    n_pairs_all = cdiv(a.n_skip_tiles, 2);
    n_tiles = n_pairs_gemm;
    K = a.H;
  } else if constexpr (KIND == kDhidden) {
    m_tiles = a.counts[1];
    n_tiles = cdiv(a.H, kTile);
    K = a.Ws;
  } else {
    m_tiles = cdiv(a.Ws, kTile);
    n_tiles = cdiv(a.H, kTile);
    K = a.T;
  }
  const int64_t n_gemm = m_tiles * n_tiles;
  const int64_t n_items =
      n_gemm + (KIND == kDlogits ? m_tiles * (n_pairs_all - n_pairs_gemm) : 0);
  const int64_t G = gridDim.x;
  const int64_t remap_end = (G % 8 == 0) ? (n_gemm / G) * G : 0;
  const int nk = (int)cdiv(K, kBK);

  const char *hp = reinterpret_cast<const char *>(a.h);
  const char *Wp = reinterpret_cast<const char *>(a.W);
  const char *Dp = reinterpret_cast<const char *>(a.D);

  for (int64_t item = blockIdx.x; item < n_items; item += G) {
    // ---------------- zero tiles of the d-logits staging ----------------
    if constexpr (KIND == kDlogits) {
      if (item >= n_gemm) {
        const int64_t z = item - n_gemm;
        const int64_t mi = z % m_tiles;
        const int64_t p = n_pairs_gemm + z / m_tiles;
        const int64_t c0 = mi * kTile;
        const int64_t c1 = (c0 + kTile < a.ld_d) ? c0 + kTile : a.ld_d;
        constexpr int kChunks = kTile / kPer;
        for (int idx = tid; idx < kTile * kChunks; idx += kThreads) {
          const int row = idx / kChunks;
          const int ch = idx - row * kChunks;
          const int64_t e = 2 * p + (row >> 7);
          if (e >= a.n_skip_tiles) continue;
          const int64_t t = (int64_t)a.tile_list[e] * kSkipTile + (row & 127);
          const int64_t col = c0 + (int64_t)ch * kPer;
          if (t < a.T && col < c1)
            *reinterpret_cast<u32x4 *>(const_cast<char *>(Dp) + (t * a.ld_d + col) * kEsz) =
                u32x4{0u, 0u, 0u, 0u};
        }
        continue;
      }
    }

    // ---------------- tile coordinates ----------------
    int64_t L = item;
    if (item < remap_end) {
      const int64_t r = item / G;
      const int64_t b = item - r * G;
      L = r * G + (b & 7) * (G >> 3) + (b >> 3);
    }
    int64_t mi, ni;
    group_map(L, m_tiles, n_tiles, a.group_m > 0 ? a.group_m : 8, mi, ni);

    int64_t span_s0 = 0, span_s1 = 0;
    if constexpr (KIND == kDhidden) {
      span_s0 = a.span_tiles[2 * mi];
      span_s1 = a.span_tiles[2 * mi + 1];
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if constexpr (KIND == kDhidden) {
      // Splits after the first continue the fp32 sum of the earlier splits: start the
      // accumulators from it, so the epilogue is a plain store.
      if (!a.first_split) {
        const int n_rows = (int)(span_s1 - span_s0);
        const int64_t n_tile = ni * kTile;
        const int n_cols = (a.H - n_tile) < kTile ? (int)(a.H - n_tile) : kTile;
        const float *base = a.dh_acc + span_s0 * a.H + n_tile;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = wm * 128 + (g << 2) + i * 32 + ((r >> 2) << 3) + (r & 3);
            const float *prow = base + (uint32_t)(row < n_rows ? row : 0) * (uint32_t)a.H;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int col = wn * 128 + (lane & 31) + j * 32;
              acc[i][j][r] = (row < n_rows && col < n_cols) ? prow[col] : 0.f;
            }
          }
      }
    }

    if constexpr (!kV2) {
    // ---------------- operand addressing ----------------
    // Uniform 64-bit bases (tile origin at K = 0) plus 32-bit per-thread byte
    // offsets.  Rows past the end of an operand are clamped onto its last row:
    // they load real data whose products only reach outputs that are never
    // stored.  Only the last K stage, when K is not a multiple of the stage,
    // zeroes out-of-range K (and clamps its addresses so nothing is read past
    // an allocation).
    //
    // Row-chunk operands (K contiguous): thread owns 16-byte chunk (tid & 7) of
    // tile rows (tid >> 3) + 32 i, offsets from one base, except the d-logits
    // token operand whose two 128-row halves come from two tiles (base0, base1).
    // Transposed operands (K = row index in memory): thread owns the kPer x kPer
    // block at K rows (lane & 7) * kPer + [0, kPer) and M chunk
    // (lane >> 3) + 8 wave (+ 32 for the second fp32 block).
    const int r_base = tid >> 3;
    const int kchunk = lane & 7;
    const char *a_base0 = nullptr, *a_base1 = nullptr, *b_base0 = nullptr, *b_base1 = nullptr;
    uint32_t a_off[8], b_off[8];
    int64_t a_ld = 0, b_ld = 0;   // bytes between K rows (transposed operands)
    if constexpr (KIND == kFwd) {
      const int64_t v0 = mi * kTile, t0 = ni * kTile;
      a_base0 = Wp + v0 * a.H * kEsz;
      a_base1 = a_base0;
      b_base0 = hp + t0 * a.H * kEsz;
      b_base1 = b_base0;
      const int64_t va = a.V - 1 - v0, tb = a.T - 1 - t0;  // last valid tile row
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = r_base + 32 * i;
        const int64_t ra_ = r < va ? r : va;
        const int64_t rb_ = r < tb ? r : tb;
        a_off[i] = (uint32_t)(ra_ * a.H * kEsz + (tid & 7) * 16);
        b_off[i] = (uint32_t)(rb_ * a.H * kEsz + (tid & 7) * 16);
      }
    } else if constexpr (KIND == kDlogits) {
      const int64_t v0 = mi * kTile;
      a_base0 = Wp + (a.v_base + v0) * a.H * kEsz;
      a_base1 = a_base0;
      const int64_t e0 = 2 * ni, e1 = 2 * ni + 1;
      const int64_t tile0 = a.tile_list[e0];
      const int64_t tile1 = (e1 < a.n_skip_tiles) ? a.tile_list[e1] : tile0;
      b_base0 = hp + tile0 * kSkipTile * a.H * kEsz;
      b_base1 = hp + tile1 * kSkipTile * a.H * kEsz;
      const int64_t va = a.Ws - 1 - v0;
      const int64_t tb0 = a.T - 1 - tile0 * kSkipTile, tb1 = a.T - 1 - tile1 * kSkipTile;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = r_base + 32 * i;
        const int64_t ra_ = r < va ? r : va;
        const int64_t rl = r & 127;
        const int64_t tb = i >= 4 ? tb1 : tb0;
        a_off[i] = (uint32_t)(ra_ * a.H * kEsz + (tid & 7) * 16);
        b_off[i] = (uint32_t)((rl < tb ? rl : tb) * a.H * kEsz + (tid & 7) * 16);
      }
    } else if constexpr (KIND == kDhidden) {
      a_base0 = Dp + span_s0 * a.ld_d * kEsz;
      a_base1 = a_base0;
      const int64_t ra_max = span_s1 - 1 - span_s0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = r_base + 32 * i;
        const int64_t ra_ = r < ra_max ? r : ra_max;
        a_off[i] = (uint32_t)(ra_ * a.ld_d * kEsz + (tid & 7) * 16);
      }
      // B = W rows of the split (K) x columns n (M chunk), transposed on load
      b_base0 = Wp + a.v_base * a.H * kEsz;
      b_ld = a.H * kEsz;
#pragma unroll
      for (int b = 0; b < 8 / kPer; ++b) {
        int64_t n = ni * kTile + ((lane >> 3) + 8 * wave + 32 * b) * kPer;
        if (n >= a.H) n = 0;
        b_off[b] = (uint32_t)(n * kEsz);
      }
    } else {
      // A = D (K = token rows) x split columns v; B = h (K = token rows) x n
      a_base0 = Dp;
      a_ld = (int64_t)a.ld_d * kEsz;
      b_base0 = hp;
      b_ld = a.H * kEsz;
#pragma unroll
      for (int b = 0; b < 8 / kPer; ++b) {
        const int64_t mch = (lane >> 3) + 8 * wave + 32 * b;
        int64_t v = mi * kTile + mch * kPer;
        if (v >= a.ld_d) v = 0;
        int64_t n = ni * kTile + mch * kPer;
        if (n >= a.H) n = 0;
        a_off[b] = (uint32_t)(v * kEsz);
        b_off[b] = (uint32_t)(n * kEsz);
      }
    }

    const bool has_tail = (K % kBK) != 0;
    // Loads never branch: in the last, partial K stage out-of-range chunks read a
    // clamped in-range address, and are replaced by zeros only when the stage is
    // written to LDS (after the MFMAs), so the loads stay in flight meanwhile.
    auto row_kok = [&](int kt) -> bool {
      return !(has_tail && kt == nk - 1) || ((int64_t)kt * kBK + (tid & 7) * kPer < K);
    };
    // ---------------- global -> registers ----------------
    auto load_rows = [&](const char *base0, const char *base1, const uint32_t (&off)[8], int kt,
                         u32x4 (&reg)[8]) {
      uint32_t kb = (uint32_t)kt * 128u;
      // out-of-range chunk: read the (aligned, in-row) chunk holding element K - 1
      if (!row_kok(kt)) kb = (uint32_t)(((K - 1) / kPer) * kPer * kEsz) - (tid & 7) * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        reg[i] = *reinterpret_cast<const u32x4 *>((i < 4 ? base0 : base1) + (uint32_t)(off[i] + kb));
    };
    auto load_tr = [&](const char *base, const uint32_t (&off)[8], int64_t ld, int kt,
                       u32x4 (&reg)[8]) {
      const char *bk = base + (int64_t)kt * kBK * ld;
      const int64_t krem = K - (int64_t)kt * kBK;  // valid K rows from this stage on
#pragma unroll
      for (int b = 0; b < 8 / kPer; ++b) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          int64_t kl = kchunk * kPer + i;
          if (kl >= krem) kl = krem - 1;  // clamp onto the last K row
          reg[b * kPer + i] =
              *reinterpret_cast<const u32x4 *>(bk + (uint32_t)(off[b] + (uint32_t)kl * (uint32_t)ld));
        }
      }
    };
    // ---------------- registers -> LDS ----------------
    auto store_rows = [&](char *dst, const u32x4 (&reg)[8], int kt) {
      const bool z = !row_kok(kt);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4 *>(dst + (r_base + 32 * i) * kRowBytes + (tid & 7) * 16) =
            z ? u32x4{0u, 0u, 0u, 0u} : reg[i];
    };
    auto store_tr = [&](char *dst, u32x4 (&reg)[8], int kt) {
      if (has_tail && kt == nk - 1) {
        const int64_t krem = K - (int64_t)kt * kBK;
#pragma unroll
        for (int b = 0; b < 8 / kPer; ++b)
#pragma unroll
          for (int i = 0; i < kPer; ++i)
            if (kchunk * kPer + i >= krem) reg[b * kPer + i] = u32x4{0u, 0u, 0u, 0u};
      }
      u32x4 tr[8];
      transpose_block(reg, tr, T{});
#pragma unroll
      for (int b = 0; b < 8 / kPer; ++b) {
        const int mch = (lane >> 3) + 8 * wave + 32 * b;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          *reinterpret_cast<u32x4 *>(dst + (mch * kPer + j) * kRowBytes + kchunk * 16) =
              tr[b * kPer + j];
      }
    };

    u32x4 ra[8], rb[8];
    auto load_stage = [&](int kt) {
      if constexpr (kATr) load_tr(a_base0, a_off, a_ld, kt, ra);
      else load_rows(a_base0, a_base1, a_off, kt, ra);
      if constexpr (kBTr) load_tr(b_base0, b_off, b_ld, kt, rb);
      else load_rows(b_base0, b_base1, b_off, kt, rb);
    };
    auto store_stage = [&](int st, int kt) {
      char *As = smem + st * 2 * kOpBytes;
      char *Bs = As + kOpBytes;
      if constexpr (kATr) store_tr(As, ra, kt);
      else store_rows(As, ra, kt);
      if constexpr (kBTr) store_tr(Bs, rb, kt);
      else store_rows(Bs, rb, kt);
    };

    load_stage(0);
    store_stage(0, 0);
    __syncthreads();
    // Fragment reads are double-buffered: the 8 LDS reads of K slice q+1 are
    // issued while the 16 MFMAs of slice q run, interleaved one read per two
    // MFMAs, so LDS latency hides behind matrix-core work.
    const int frag_row = lane & 31;
    const int a_frag = (wm * 128 + frag_row) * kRowBytes + g * 16;
    const int b_frag = (wn * 128 + frag_row) * kRowBytes + g * 16;
    // reads in the order the MFMAs consume them: A0, B0..B3, A1..A3
    auto read_frags = [&](const char *As, const char *Bs, int q, u32x4 (&fa)[4], u32x4 (&fb)[4]) {
      fa[0] = *reinterpret_cast<const u32x4 *>(As + a_frag + q * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const u32x4 *>(Bs + b_frag + j * 32 * kRowBytes + q * 32);
#pragma unroll
      for (int i = 1; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4 *>(As + a_frag + i * 32 * kRowBytes + q * 32);
    };
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < nk) load_stage(kt + 1);
      const char *As = smem + st * 2 * kOpBytes;
      const char *Bs = As + kOpBytes;
      u32x4 fa[2][4], fb[2][4];
      read_frags(As, Bs, 0, fa[0], fb[0]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < 3) read_frags(As, Bs, q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) Mma<T>::run(acc[i][j], fa[q & 1][i], fb[q & 1][j]);
        if (q < 3) {
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kt + 1 < nk) store_stage(st ^ 1, kt + 1);
      __syncthreads();
    }

    } else {
      // ================= bf16: LDS-direct loads into a kNS-stage ring =================
      // Each stage holds 32 K elements of both operands.  Loads go straight from
      // global memory into LDS (buffer_load ... lds: lane l of a wave writes 16 bytes
      // at the instruction's LDS base + 16 l), kNS-1 stages ahead of the MFMAs, so no
      // VGPRs stage the data and no LDS stores are issued.  Buffer descriptors bound
      // every operand: rows past its end read as zero.
      //
      // Row-form operands (K contiguous in memory: W, h, the d-logits rows) are stored
      // as [256 rows][4 chunks of 16 B]; logical chunk c of row r sits at position
      // c ^ swz_row(r), which spreads the 16 rows read together by an MFMA fragment
      // read over distinct banks.  Transposed operands (K = the row index in memory:
      // W for dHidden, the d-logits and h for dWeight) are stored as loaded, as
      // [32 K rows][32 chunks of 16 B along M], chunk c of K row k at c ^ (4 (k % 4)),
      // and turned into K-contiguous fragments by ds_read_b64_tr_b16: within a group
      // of 16 lanes, lane i reads 4 consecutive M elements of K row kb + i / 4 at
      // column mb + 4 (i % 4), and lane j receives K rows kb..kb+3 of column mb + j.
      constexpr bool kATrV = (KIND == kDweight);
      constexpr bool kBTrV = (KIND == kDhidden || KIND == kDweight);
      constexpr int kLPS = 8;  // load instructions per stage per wave (4 per operand)
      const int nkv = (int)cdiv(K, 32);
      const bool ktail = (K % 32) != 0;

      // row-form: resources for tile rows [0,128) and [128,256); a wave loads one half only
      __amdgpu_buffer_rsrc_t ra0, ra1, rb0, rb1;
      uint32_t a_vo[4], b_vo[4];            // per load instruction: this lane's byte offset at k = 0
      uint8_t a_ck[4], b_ck[4];             // row-form: this lane's logical K chunk per instruction
      const char *a_tb = nullptr, *b_tb = nullptr;  // transposed: (k = 0, m = tile origin)
      int64_t a_ldb = 0, b_ldb = 0;                 // transposed: bytes per K row

      auto swz_row = [](int r) { return ((r >> 1) & 2) | (((r >> 1) & 1) ^ ((r >> 3) & 1)); };
      const int swz_lane = swz_row(lane & 31);  // same for every fragment row of this lane
      auto rsrc = [](const char *base, int64_t bytes) {
        const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, (int)n, 0x00020000);
      };
      // Row-form source: rows of `ld_bytes` bytes; tile rows [0,128) start at base0
      // with n0 valid rows, tile rows [128,256) at base1 with n1 valid rows.
      auto setup_rows = [&](const char *base0, int64_t n0, const char *base1, int64_t n1,
                            int64_t ld_bytes, __amdgpu_buffer_rsrc_t &r0, __amdgpu_buffer_rsrc_t &r1,
                            uint32_t (&vo)[4],
                            uint8_t (&ck)[4]) {
        r0 = rsrc(base0, n0 * ld_bytes);
        r1 = rsrc(base1, n1 * ld_bytes);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int row = 16 * (4 * wave + n) + (lane >> 2);  // tile row this lane loads
          const int c = (lane & 3) ^ swz_row(row);
          ck[n] = (uint8_t)c;
          vo[n] = (uint32_t)((int64_t)(row & 127) * ld_bytes) + (uint32_t)(c * 16);
        }
      };
      // Transposed source: element (k, m) at base + k * ld_bytes + m * 2, tile origin m0.
      auto setup_tr = [&](int64_t m0, int64_t ld_bytes, uint32_t (&vo)[4]) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int krow = 8 * wave + 2 * n + (lane >> 5);
          const int c = (lane & 31) ^ (4 * (krow & 3));
          vo[n] = (uint32_t)((int64_t)krow * ld_bytes + m0 * 2 + c * 16);
        }
      };

      if constexpr (KIND == kFwd) {
        const int64_t v0 = mi * kTile, t0 = ni * kTile;
        const int64_t ldb = a.H * 2;
        const int64_t nv = a.V - v0, nt = a.T - t0;
        setup_rows(Wp + v0 * ldb, nv < 128 ? nv : 128, Wp + (v0 + 128) * ldb, nv - 128,
                   ldb, ra0, ra1, a_vo, a_ck);
        setup_rows(hp + t0 * ldb, nt < 128 ? nt : 128, hp + (t0 + 128) * ldb, nt - 128,
                   ldb, rb0, rb1, b_vo, b_ck);
      } else if constexpr (KIND == kDlogits) {
        const int64_t v0 = mi * kTile;
        const int64_t ldb = a.H * 2;
        const int64_t nv = a.Ws - v0;
        setup_rows(Wp + (a.v_base + v0) * ldb, nv < 128 ? nv : 128,
                   Wp + (a.v_base + v0 + 128) * ldb, nv - 128, ldb, ra0, ra1, a_vo, a_ck);
        const int64_t e1 = 2 * ni + 1;
        const int64_t tile0 = a.tile_list[2 * ni];
        const int64_t tile1 = (e1 < a.n_skip_tiles) ? a.tile_list[e1] : -1;
        const int64_t n0 = a.T - tile0 * kSkipTile;
        const int64_t n1 = tile1 >= 0 ? a.T - tile1 * kSkipTile : 0;
        setup_rows(hp + tile0 * kSkipTile * ldb, n0 < 128 ? n0 : 128,
                   hp + (tile1 >= 0 ? tile1 : 0) * kSkipTile * ldb, n1 < 128 ? n1 : 128, ldb, rb0,
                   rb1, b_vo, b_ck);
      } else if constexpr (KIND == kDhidden) {
        const int64_t ldb = (int64_t)a.ld_d * 2;
        const int64_t nr = span_s1 - span_s0;
        setup_rows(Dp + span_s0 * ldb, nr < 128 ? nr : 128, Dp + (span_s0 + 128) * ldb, nr - 128,
                   ldb, ra0, ra1, a_vo, a_ck);
        b_tb = Wp + a.v_base * a.H * 2;
        b_ldb = a.H * 2;
        setup_tr(ni * kTile, b_ldb, b_vo);
      } else {
        a_tb = Dp;
        a_ldb = (int64_t)a.ld_d * 2;
        setup_tr(mi * kTile, a_ldb, a_vo);
        b_tb = hp;
        b_ldb = a.H * 2;
        setup_tr(ni * kTile, b_ldb, b_vo);
      }

      // Loads of stage s into ring buffer s % kNS, one operand at a time (4 instructions
      // per wave each).  Stages past the last one are still issued, with zero-size
      // descriptors (they read nothing and write zeros into a buffer nobody reads
      // any more), so the loop body has no branch and the vmcnt targets are constant.
      const __amdgpu_buffer_rsrc_t rnull = rsrc(Wp, 0);
      auto issue_a = [&](int s) {
        char *lb = smem + (s % kNS) * kStage;
        const bool live = s < nkv;
        if constexpr (kATrV) {
          const __amdgpu_buffer_rsrc_t r =
              live ? rsrc(a_tb + (int64_t)s * 32 * a_ldb, (K - (int64_t)s * 32) * a_ldb) : rnull;
#pragma unroll
          for (int n = 0; n < 4; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lb + (8 * wave + 2 * n) * 512, 16, a_vo[n], 0, 0, 0);
        } else {
          const __amdgpu_buffer_rsrc_t r = live ? ((wave >> 1) ? ra1 : ra0) : rnull;
#pragma unroll
          for (int n = 0; n < 4; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lb + (4 * wave + n) * 1024, 16, a_vo[n], s * 64, 0, 0);
        }
      };
      auto issue_b = [&](int s) {
        char *lbb = smem + (s % kNS) * kStage + kOpStage;
        const bool live = s < nkv;
        if constexpr (kBTrV) {
          const __amdgpu_buffer_rsrc_t r =
              live ? rsrc(b_tb + (int64_t)s * 32 * b_ldb, (K - (int64_t)s * 32) * b_ldb) : rnull;
#pragma unroll
          for (int n = 0; n < 4; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lbb + (8 * wave + 2 * n) * 512, 16, b_vo[n], 0, 0, 0);
        } else {
          const __amdgpu_buffer_rsrc_t r = live ? ((wave >> 1) ? rb1 : rb0) : rnull;
#pragma unroll
          for (int n = 0; n < 4; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lbb + (4 * wave + n) * 1024, 16, b_vo[n], s * 64, 0, 0);
        }
      };
      // Last, partial K stage of a row-form operand: its chunks past K were read from
      // the next row (or as zeros); overwrite them with zeros once this wave's loads
      // of the stage have landed.
      auto fix_tail = [&](int s) {
        if (!(ktail && s == nkv - 1)) return;
        char *lb = smem + (s % kNS) * kStage;
        if constexpr (!kATrV) {
#pragma unroll
          for (int n = 0; n < 4; ++n)
            if ((int64_t)s * 32 + a_ck[n] * 8 >= K)
              *reinterpret_cast<u32x4 *>(lb + (4 * wave + n) * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (!kBTrV) {
#pragma unroll
          for (int n = 0; n < 4; ++n)
            if ((int64_t)s * 32 + b_ck[n] * 8 >= K)
              *reinterpret_cast<u32x4 *>(lb + kOpStage + (4 * wave + n) * 1024 + lane * 16) =
                  u32x4{0u, 0u, 0u, 0u};
        }
      };
      // s_waitcnt immediates (gfx9): vmcnt in [3:0] and [15:14], expcnt [6:4] = 7 and
      // lgkmcnt [11:8] = 15 (no wait on those)
      constexpr int kVm16 = 0x0f70 | (16 & 15) | ((16 >> 4) << 14);  // <= 16 loads in flight
      constexpr int kVm12 = 0x0f70 | (12 & 15) | ((12 >> 4) << 14);  // <= 12 loads in flight
      constexpr int kLgkm0 = 0xc07f;                                 // lgkmcnt(0) only
      static_assert(kNS == 4, "the vmcnt targets below assume a 4-stage ring");

      // ---- fragment reads ----
      const int G16 = lane >> 4, h16 = G16 & 1, g16 = G16 >> 1, li = lane & 15;
      auto read_rowform = [&](const char *op, int wbase, int i, int q) -> u32x4 {
        const int R = wbase + 32 * i + (lane & 31);
        return *reinterpret_cast<const u32x4 *>(op + R * 64 + (((2 * q + g) ^ swz_lane) << 4));
      };
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      auto read_tr = [&](const char *op, int wbase, int i, int q) -> u32x4 {
        const int m = wbase + 32 * i + 16 * h16 + 4 * (li & 3);
        const int sw = 4 * ((li >> 2) & 3);
        const int col = ((((m >> 3) ^ sw)) << 4) + ((m & 7) << 1);
        const int k0 = 16 * q + 8 * g16 + (li >> 2);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3))) *)(op + k0 * 512 + col));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 __attribute__((address_space(3))) *)(op + (k0 + 4) * 512 + col));
        // 4 x b16 in two dwords, element 0 in the low half: already the fragment layout
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
      };
      auto read_frags2 = [&](int s, int q, u32x4 (&fa)[4], u32x4 (&fb)[4]) {
        const char *lb = smem + (s % kNS) * kStage;
        auto ra_ = [&](int i) { return kATrV ? read_tr(lb, wm * 128, i, q) : read_rowform(lb, wm * 128, i, q); };
        auto rb_ = [&](int j) {
          return kBTrV ? read_tr(lb + kOpStage, wn * 128, j, q) : read_rowform(lb + kOpStage, wn * 128, j, q);
        };
        fa[0] = ra_(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = rb_(j);
#pragma unroll
        for (int i = 1; i < 4; ++i) fa[i] = ra_(i);
      };
      constexpr int kReads = (kATrV ? 8 : 4) + (kBTrV ? 8 : 4);  // LDS reads per K slice
      constexpr bool kAnyTr = kATrV || kBTrV;
      constexpr int kVmemPerHalf = kAnyTr ? 8 : 4;  // loads spread over one half-stage
      // 16 MFMAs of one K slice, with the next slice's LDS reads and (optionally) 4
      // global->LDS loads spread between them
      auto mma_slice = [&](const u32x4 (&fa)[4], const u32x4 (&fb)[4], bool interleave, bool vmem) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
        if (interleave) {
#pragma unroll
          for (int x = 0; x < kReads; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // one LDS read
            if (vmem && x < kVmemPerHalf) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a load
            __builtin_amdgcn_sched_group_barrier(0x008, kReads <= 8 ? 2 : 1, 0);   // MFMA(s)
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      };

      // ---- prologue: stages 0 .. kNS-2 in flight, stage 0 visible ----
#pragma unroll
      for (int s = 0; s < kNS - 1; ++s) {
        issue_a(s);
        issue_b(s);
      }
      __builtin_amdgcn_s_waitcnt(kVm16);  // this wave's stage-0 loads have landed
      fix_tail(0);
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      u32x4 F0a[4], F0b[4], F1a[4], F1b[4];
      read_frags2(0, 0, F0a, F0b);
      __builtin_amdgcn_sched_barrier(0);

      // Stages 0 .. nkv-2: each iteration also brings stage kt+1 into view and issues
      // stage kt+3 (A half before the barrier, B half after it).  The last stage is
      // peeled so the loop body is one straight MFMA path.
      for (int kt = 0; kt + 1 < nkv; ++kt) {
        // Row-form kernels spread the 8 loads of stage kt+3 over both halves (A before
        // the barrier, B after it); the transposed-operand kernels are more latency
        // bound and issue both halves before the barrier, spread over the first half.
        issue_a(kt + kNS - 1);  // into the buffer stage kt-1 used
        if constexpr (kAnyTr) issue_b(kt + kNS - 1);
        read_frags2(kt, 1, F1a, F1b);
        mma_slice(F0a, F0b, true, true);
        // loads after stage kt+1's: A,B of stage kt+2 and A (and B) of stage kt+3
        __builtin_amdgcn_s_waitcnt(kAnyTr ? kVm16 : kVm12);
        fix_tail(kt + 1);
        __builtin_amdgcn_s_waitcnt(kLgkm0);  // this wave's reads of stage kt done
        __builtin_amdgcn_s_barrier();
        if constexpr (!kAnyTr) issue_b(kt + kNS - 1);
        read_frags2(kt + 1, 0, F0a, F0b);
        mma_slice(F1a, F1b, true, !kAnyTr);
      }
      read_frags2(nkv - 1, 1, F1a, F1b);
      mma_slice(F0a, F0b, true, false);
      mma_slice(F1a, F1b, false, false);
      __builtin_amdgcn_s_waitcnt(0x0f70);  // drain the trailing loads (they target free buffers)
      __syncthreads();  // every wave is done with the ring before epilogues reuse LDS
    }

    // ---------------- epilogues ----------------
    // acc[i][j][r] holds tile row  wm*128 + i*32 + 8*(r/4) + 4*g + (r%4)
    //               and tile col  wn*128 + j*32 + (lane % 32).
    // Indices below are tile-local 32-bit; tile origins are uniform.
    const int row0 = wm * 128 + (g << 2);   // + i*32 + 8*(r/4) + (r%4)
    const int col0 = wn * 128 + (lane & 31);  // + j*32
    if constexpr (KIND == kFwd) {
      const int64_t v_tile = mi * kTile;
      const int n_rows = (a.V - v_tile) < kTile ? (int)(a.V - v_tile) : kTile;  // valid vocab rows
      const bool full = n_rows == kTile;
      const int64_t t_tile = ni * kTile;
      float4 *xch = reinterpret_cast<float4 *>(smem);
      float st_M[4], st_s[4], st_u[4], st_zy[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + j * 32;
        const int64_t t = t_tile + col;
        // target row local to this tile, or -1
        int yl = -1;
        if (t < a.T) {
          const int64_t yd = a.targets[t] - v_tile;
          yl = (yd >= 0 && yd < kTile) ? (int)yd : -1;
        }
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + i * 32 + ((r >> 2) << 3) + (r & 3);
            if (full || row < n_rows) mx = fmaxf(mx, acc[i][j][r]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float s = 0.f, u = 0.f, zy = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + i * 32 + ((r >> 2) << 3) + (r & 3);
            const float z = acc[i][j][r];
            if (full || row < n_rows) {
              const float d = z - mx;
              const float e = __expf(d);
              s += e;
              u += e * d;
            }
            if (row == yl) zy = z;
          }
        s += __shfl_xor(s, 32);
        u += __shfl_xor(u, 32);
        zy = fmaxf(zy, __shfl_xor(zy, 32));
        st_M[j] = mx;
        st_s[j] = s;
        st_u[j] = u;
        st_zy[j] = zy;
        if (wm == 1 && lane < 32) xch[col] = make_float4(mx, s, u, zy);
      }
      __syncthreads();
      if (wm == 0 && lane < 32) {
        float4 *out = reinterpret_cast<float4 *>(a.part) + mi * a.T + t_tile;
        const int n_cols = (a.T - t_tile) < kTile ? (int)(a.T - t_tile) : kTile;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = col0 + j * 32;
          const float4 o = xch[col];
          float M = st_M[j], s = st_s[j], u = st_u[j];
          merge_state(M, s, u, o.x, o.y, o.z);
          const float zy = fmaxf(st_zy[j], o.w);
          if (col < n_cols) out[col] = make_float4(M, s, u, zy);
        }
      }
    } else if constexpr (KIND == kDlogits) {
      const int64_t v_tile = mi * kTile;                 // split-local first column
      const int n_live = (a.Ws - v_tile) < kTile ? (int)(a.Ws - v_tile) : kTile;
      const int n_cols = (a.ld_d - v_tile) < kTile ? (int)(a.ld_d - v_tile) : kTile;
      T *Dt = reinterpret_cast<T *>(a.D) + v_tile;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + j * 32;
        const int64_t e = 2 * ni + (col >> 7);
        const int64_t tile = (e < a.n_skip_tiles) ? a.tile_list[e] : -1;
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
        const int lim = act ? n_live : 0;   // columns >= lim are stored as 0
        T *drow = Dt + t * a.ld_d;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c0 = row0 + i * 32 + q * 8;  // first of 4 consecutive columns
            float d[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float z = acc[i][j][4 * q + c];
              const float p = __expf(z - lse_t);
              const float val = ga * ((c0 + c == yl ? 1.f : 0.f) - p) + gb * p * (ez - z);
              d[c] = (c0 + c < lim) ? val : 0.f;
            }
            if (tok && c0 < n_cols) store4(drow + c0, d[0], d[1], d[2], d[3]);
          }
      }
    } else if constexpr (KIND == kDhidden) {
      const int n_rows = (int)(span_s1 - span_s0);
      const int64_t n_tile = ni * kTile;
      const int n_cols = (a.H - n_tile) < kTile ? (int)(a.H - n_tile) : kTile;
      float *base = a.dh_acc + span_s0 * a.H + n_tile;
      const uint32_t ldh = (uint32_t)a.H;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + i * 32 + ((r >> 2) << 3) + (r & 3);
          if (row >= n_rows) continue;
          float *prow = base + (uint32_t)row * ldh;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = col0 + j * 32;
            if (col < n_cols) prow[col] = acc[i][j][r];
          }
        }
    } else {
      const int64_t v_tile = mi * kTile;
      const int n_rows = (a.Ws - v_tile) < kTile ? (int)(a.Ws - v_tile) : kTile;
      const int64_t n_tile = ni * kTile;
      const int n_cols = (a.H - n_tile) < kTile ? (int)(a.H - n_tile) : kTile;
      T *base = reinterpret_cast<T *>(a.dW) + (a.v_base + v_tile) * a.H + n_tile;
      const uint32_t ldw = (uint32_t)a.H;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + i * 32 + ((r >> 2) << 3) + (r & 3);
          if (row >= n_rows) continue;
          T *prow = base + (uint32_t)row * ldw;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = col0 + j * 32;
            if (col < n_cols) store1(prow + col, acc[i][j][r]);
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
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, GemmKind kind, const GemmArgs &a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  return dtype == 1 ? launch_t<uint16_t>(kind, a, grid, st) : launch_t<float>(kind, a, grid, st);
}

}  // namespace flh
