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
// 8 m-tiles, m fastest: 32 consecutive ids form an 8 x 4 block.
__device__ __forceinline__ void group_map(int64_t L, int64_t m_tiles, int64_t n_tiles,
                                          int64_t &mi, int64_t &ni) {
  const int64_t per_group = 8 * n_tiles;
  const int64_t g = L / per_group;
  const int64_t r = L - g * per_group;
  const int64_t first = g * 8;
  const int64_t gm = (m_tiles - first) < 8 ? (m_tiles - first) : 8;
  mi = first + r % gm;
  ni = r / gm;
}

template <typename T, int KIND>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  constexpr int kPer = Elt<T>::kPer;       // elements per 16-byte chunk
  constexpr int kBK = 128 / sizeof(T);     // K elements per stage
  constexpr bool kATr = (KIND == kDweight);
  constexpr bool kBTr = (KIND == kDhidden || KIND == kDweight);
  constexpr int64_t kEsz = sizeof(T);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    group_map(L, m_tiles, n_tiles, mi, ni);

    int64_t span_s0 = 0, span_s1 = 0;
    if constexpr (KIND == kDhidden) {
      span_s0 = a.span_tiles[2 * mi];
      span_s1 = a.span_tiles[2 * mi + 1];
    }

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

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

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
            if (col < n_cols) prow[col] = a.first_split ? acc[i][j][r] : prow[col] + acc[i][j][r];
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
