// Small, memory-bound kernels around the contractions:
//
//   spans    loss mask -> tile bitmap, ordered active spans, span count, active
//            count (SkyRL #2376, "How it works": one builder derives the forward
//            active mask and the backward spans; Bugbot "Overview": runs of the
//            RL loss mask coalesced across gaps <= 128).  Built on the device.
//   lists    bitmap + spans -> the backward's work lists: token tiles (active
//            ones first, so d-logits workgroups pair up active tiles) and
//            span-local row tiles for the hidden-gradient projection.
//   combine  per-tile softmax states -> logprob, entropy, lse per token.
//   finalize fp32 hidden-gradient accumulator -> output dtype, inactive rows +0,
//            NaN rows for active tokens the metadata does not cover.
//
// spans and lists run as one workgroup of 1024 threads: the mask is at most a
// few hundred KiB, so a single pass through L2 is far cheaper than a multi-kernel
// scan, and nothing has to be synchronised with the host.
#include <hip/hip_runtime.h>

#include "flh_internal.h"

namespace flh {
namespace {

constexpr int kBlock = 1024;

// Inclusive scans over the 1024 threads of the block (Hillis-Steele in LDS).
template <typename V, typename Op>
__device__ V block_scan(V v, V *sh, Op op) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kBlock; off <<= 1) {
    V x = v;
    if (tid >= off) x = op(sh[tid - off], v);
    __syncthreads();
    v = x;
    sh[tid] = v;
    __syncthreads();
  }
  return v;
}

struct AddOp {
  __device__ int64_t operator()(int64_t a, int64_t b) const { return a + b; }
};
struct MaxOp {
  __device__ int64_t operator()(int64_t a, int64_t b) const { return a > b ? a : b; }
};

__global__ __launch_bounds__(kBlock) void spans_kernel(const uint8_t *__restrict__ mask, int64_t T,
                                                       int32_t G, int32_t tile_m, int64_t cap,
                                                       int32_t *__restrict__ spans,
                                                       int32_t *__restrict__ num_spans,
                                                       uint32_t *__restrict__ bits,
                                                       int32_t *__restrict__ active_count) {
  __shared__ int64_t sh[kBlock];
  const int tid = threadIdx.x;
  const int64_t chunk = (T + kBlock - 1) / kBlock;
  const int64_t c0 = (tid * chunk < T) ? tid * chunk : T;
  const int64_t c1 = (c0 + chunk < T) ? c0 + chunk : T;

  // pass 1: active count, first and last active token of the chunk
  int64_t cnt = 0, first = -1, last = -1;
  for (int64_t t = c0; t < c1; ++t) {
    if (mask[t]) {
      ++cnt;
      if (first < 0) first = t;
      last = t;
    }
  }
  block_scan(cnt, sh, AddOp());
  const int64_t A = sh[kBlock - 1];
  __syncthreads();
  // last active token before this chunk (-1 if none): exclusive max-scan of `last`
  block_scan(last, sh, MaxOp());
  const int64_t prev = (tid > 0) ? sh[tid - 1] : -1;
  __syncthreads();
  // first active token after this chunk (-1 if none): a max-scan of -first over
  // the threads in reverse order (position p holds thread kBlock-1-p); "no active
  // token" is INT64_MIN, neutral for max.
  sh[kBlock - 1 - tid] = (first >= 0) ? -first : INT64_MIN;
  __syncthreads();
  const int64_t rkey = sh[tid];
  __syncthreads();
  block_scan(rkey, sh, MaxOp());
  // sh[p] = max of -first over threads >= kBlock-1-p; threads after tid end at
  // position kBlock-2-tid.
  const int64_t after_pos = kBlock - 2 - tid;
  const int64_t after_key = (after_pos >= 0) ? sh[after_pos] : INT64_MIN;
  const int64_t next = (after_key == INT64_MIN) ? -1 : -after_key;
  __syncthreads();

  // pass 2: span starts in this chunk
  int64_t starts = 0;
  {
    int64_t pv = prev;
    for (int64_t t = c0; t < c1; ++t) {
      if (mask[t]) {
        if (pv < 0 || t - pv - 1 > (int64_t)G) ++starts;
        pv = t;
      }
    }
  }
  const int64_t st_incl = block_scan(starts, sh, AddOp());
  const int64_t total = sh[kBlock - 1];
  __syncthreads();
  int64_t k = st_incl - starts;  // global index of the next span to start

  // pass 3: emit starts and ends
  {
    int64_t pv = prev;
    for (int64_t t = c0; t < c1; ++t) {
      if (mask[t]) {
        if (pv < 0 || t - pv - 1 > (int64_t)G) {
          if (pv >= c0 && k - 1 < cap) spans[2 * (k - 1) + 1] = (int32_t)(pv + 1);
          if (k < cap) spans[2 * k] = (int32_t)t;
          ++k;
        }
        pv = t;
      }
    }
    if (last >= 0 && (next < 0 || next - last - 1 > (int64_t)G)) {
      if (k - 1 < cap) spans[2 * (k - 1) + 1] = (int32_t)(last + 1);
    }
  }

  // tile bitmap: one wave covers 64 consecutive tiles -> two words
  const int64_t n_tiles = (T + tile_m - 1) / tile_m;
  const int64_t n_words = (n_tiles + 31) / 32;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int64_t base = 0; base < n_tiles; base += kBlock) {
    const int64_t tile = base + wave * 64 + lane;
    int flag = 0;
    if (tile < n_tiles) {
      const int64_t t0 = tile * tile_m;
      const int64_t t1 = (t0 + tile_m < T) ? t0 + tile_m : T;
      for (int64_t t = t0; t < t1 && !flag; ++t) flag = mask[t] != 0;
    }
    const uint64_t ballot = __ballot(flag);
    const int64_t w0 = (base + wave * 64) / 32;
    if (lane == 0 && w0 < n_words) bits[w0] = (uint32_t)(ballot & 0xffffffffu);
    if (lane == 0 && w0 + 1 < n_words) bits[w0 + 1] = (uint32_t)(ballot >> 32);
  }

  if (tid == 0) {
    *num_spans = (int32_t)total;
    *active_count = (int32_t)A;
  }
}

__global__ __launch_bounds__(kBlock) void lists_kernel(int64_t T, const uint32_t *__restrict__ bits,
                                                       const int32_t *__restrict__ spans,
                                                       const int32_t *__restrict__ num_spans,
                                                       int64_t span_cap, int32_t *__restrict__ tile_list,
                                                       int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ span_tiles,
                                                       int64_t span_tile_cap,
                                                       uint32_t *__restrict__ covered) {
  __shared__ int64_t sh[kBlock];
  const int tid = threadIdx.x;
  const int64_t n_tiles = (T + kSkipTile - 1) / kSkipTile;
  auto active = [&](int64_t i) -> int64_t {
    return bits ? (int64_t)((bits[i >> 5] >> (i & 31)) & 1u) : 1;
  };

  // number of active token tiles
  int64_t c = 0;
  for (int64_t i = tid; i < n_tiles; i += kBlock) c += active(i);
  block_scan(c, sh, AddOp());
  const int64_t n_act = sh[kBlock - 1];
  __syncthreads();

  // stable partition: active tiles ascending, then inactive tiles ascending
  int64_t run_a = 0, run_i = 0;
  for (int64_t base = 0; base < n_tiles; base += kBlock) {
    const int64_t i = base + tid;
    const int64_t valid = i < n_tiles ? 1 : 0;
    const int64_t f = valid ? active(i) : 0;
    const int64_t nf = valid - f;
    const int64_t pa = block_scan(f, sh, AddOp());
    const int64_t tot_a = sh[kBlock - 1];
    __syncthreads();
    const int64_t pi = block_scan(nf, sh, AddOp());
    const int64_t tot_i = sh[kBlock - 1];
    __syncthreads();
    if (valid) {
      if (f) tile_list[run_a + pa - 1] = (int32_t)i;
      else tile_list[n_act + run_i + pi - 1] = (int32_t)i;
    }
    run_a += tot_a;
    run_i += tot_i;
  }

  // Spans as the kernels use them: the count clamped to [0, span_cap] and every span
  // to 0 <= start <= end <= T, so that metadata that does not belong to this call
  // (built from another mask, or never built) cannot send a launch outside its rows.
  int64_t ns = spans ? (int64_t)(*num_spans) : 1;
  if (ns > span_cap && spans) ns = span_cap;
  if (ns < 0) ns = 0;
  auto span_at = [&](int64_t k, int64_t &s, int64_t &e) {
    if (!spans) {
      s = 0;
      e = T;
      return;
    }
    s = spans[2 * k];
    e = spans[2 * k + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
  };

  // Tokens the metadata covers, one bit per token: inside a span and in a token tile
  // whose bit is set.  With metadata built from this call's mask every active token is
  // covered; the finalize step gives an active token that is not a NaN hidden-gradient
  // row, so inconsistent metadata fails loudly instead of leaving stale or zero rows.
  if (covered) {
    const int64_t n_cw = (T + 31) / 32;
    for (int64_t w = tid; w < n_cw; w += kBlock) {
      const int64_t t0 = w * 32;
      int64_t lo = 0, hi = ns;  // first span whose end is past t0 (ends ascend)
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        int64_t s, e;
        span_at(mid, s, e);
        if (e <= t0) lo = mid + 1;
        else hi = mid;
      }
      int64_t k = lo, ks = 0, ke = 0;
      if (k < ns) span_at(k, ks, ke);
      uint32_t word = 0u;
      for (int b = 0; b < 32 && t0 + b < T; ++b) {
        const int64_t t = t0 + b;
        while (k < ns && ke <= t) {
          ++k;
          if (k < ns) span_at(k, ks, ke);
        }
        const bool in_span = k < ns && ks <= t;
        if (in_span && active(t / kSkipTile)) word |= 1u << b;
      }
      covered[w] = word;
    }
  }

  // span pieces of at most kSpanPiece rows, starting at each span start (span order)
  int64_t run = 0;
  for (int64_t base = 0; base < ns; base += kBlock) {
    const int64_t k = base + tid;
    int64_t s = 0, e = 0;
    if (k < ns) span_at(k, s, e);
    const int64_t ntl = (e > s) ? (e - s + kSpanPiece - 1) / kSpanPiece : 0;
    const int64_t incl = block_scan(ntl, sh, AddOp());
    const int64_t tot = sh[kBlock - 1];
    __syncthreads();
    for (int64_t j = 0; j < ntl; ++j) {
      const int64_t idx = run + incl - ntl + j;
      if (idx < span_tile_cap) {
        const int64_t r0 = s + j * kSpanPiece;
        span_tiles[2 * idx] = (int32_t)r0;
        span_tiles[2 * idx + 1] = (int32_t)((r0 + kSpanPiece < e) ? r0 + kSpanPiece : e);
      }
    }
    run += tot;
  }
  if (tid == 0) {
    counts[0] = (int32_t)n_act;
    const int64_t pieces = run < span_tile_cap ? run : span_tile_cap;
    counts[1] = (int32_t)((pieces + kPiecesPerTile - 1) / kPiecesPerTile);  // hidden-gradient tiles
    counts[2] = (int32_t)pieces;
  }
}

// The value of an OCP E4M3 code as fp32 (exact): sign bit 7, exponent bits 6..3 with
// bias 7, mantissa bits 2..0; exponent 0 is m/8 * 2^-6; code x1111111 is NaN; no
// infinities.  For a normal code the fp32 pattern is the code's exponent and mantissa
// moved up by 20 bits plus (127 - 7) in the exponent field.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t em = c & 0x7fu;
  const float mag = em >= 8u ? __uint_as_float((em << 20) + (120u << 23)) : (float)em * 0.001953125f;
  return em == 0x7fu ? __uint_as_float(0x7fc00000u) : __uint_as_float(__float_as_uint(mag) | sign);
}

// bits: NULL, or the tile bitmap of a forward over active 128-token tiles only; tokens
// of the other tiles get 0 for all three outputs.
__device__ __forceinline__ bool tile_skipped(const uint32_t *bits, int64_t t) {
  if (!bits) return false;
  const int64_t i = t / kSkipTile;
  return ((bits[i >> 5] >> (i & 31)) & 1u) == 0;
}

// Merge of two (max, sum e^(z - max), sum e^(z - max) (z - max)) states into the first.
__device__ __forceinline__ void merge_state(float &M, float &s, float &u, float M2, float s2, float u2) {
  const float ninf = -__builtin_huge_valf();
  const float Mn = fmaxf(M, M2);
  if (Mn == ninf) return;
  const bool e1 = (M == ninf), e2 = (M2 == ninf);
  const float c1 = e1 ? 0.f : __expf(M - Mn);
  const float c2 = e2 ? 0.f : __expf(M2 - Mn);
  const float un = (e1 ? 0.f : c1 * (u + s * (M - Mn))) + (e2 ? 0.f : c2 * (u2 + s2 * (M2 - Mn)));
  s = (e1 ? 0.f : s * c1) + (e2 ? 0.f : s2 * c2);
  u = un;
  M = Mn;
}

// Merge of the per-(vocabulary tile, token) softmax states into lse, entropy and
// logprob = z_y - lse.  A workgroup of kCombWaves waves takes 64 consecutive tokens;
// wave w merges the states of vocabulary tiles w, w + kCombWaves, ... (one coalesced
// 1 KiB read across the wave per tile), then the first wave merges the waves' states of
// each token through LDS in wave order, so the result is the same on every run.
constexpr int kCombWaves = 16;
__global__ __launch_bounds__(64 * kCombWaves) void combine_kernel(int64_t T, int64_t V,
                                                                  const float4 *__restrict__ part,
                                                                  const uint32_t *__restrict__ bits,
                                                                  float *__restrict__ logprob,
                                                                  float *__restrict__ entropy,
                                                                  float *__restrict__ lse) {
  __shared__ float4 st[kCombWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 64 + lane;
  const int64_t tc = t < T ? t : T - 1;  // rows past T read the last token's states
  const int64_t n_vt = (V + kTile - 1) / kTile;
  float M = -__builtin_huge_valf(), s = 0.f, u = 0.f;
#pragma unroll 4
  for (int64_t vt = w; vt < n_vt; vt += kCombWaves) {
    const float4 p = part[vt * T + tc];
    merge_state(M, s, u, p.x, p.y, p.z);
  }
  st[w][lane] = make_float4(M, s, u, 0.f);
  __syncthreads();
  if (w != 0 || t >= T) return;
  if (tile_skipped(bits, t)) {
    lse[t] = 0.f;
    entropy[t] = 0.f;
    logprob[t] = 0.f;
    return;
  }
  M = st[0][lane].x;
  s = st[0][lane].y;
  u = st[0][lane].z;
#pragma unroll
  for (int k = 1; k < kCombWaves; ++k) {
    const float4 q = st[k][lane];
    merge_state(M, s, u, q.x, q.y, q.z);
  }
  const float ls = __logf(s);
  const float l = M + ls;
  lse[t] = l;
  entropy[t] = ls - u / s;
  logprob[t] -= l;  // holds the target's logit z_y (NaN for a target outside [0, V))
}

// The target's logit z_y = h[t] . W[y_t], one wavefront per token: each lane takes
// 16-byte chunks of both rows, fp32 products and sums, then a butterfly over the wave.
// Written to out[t] (NaN for a target outside [0, V)).  E = uint8_t: E4M3 codes, whose
// values' dot product is multiplied by zscale.
template <typename E>
__global__ __launch_bounds__(256) void target_logit_kernel(int64_t T, int64_t H, int64_t V,
                                                           const E *__restrict__ h,
                                                           const E *__restrict__ W,
                                                           const int64_t *__restrict__ targets,
                                                           const uint32_t *__restrict__ bits,
                                                           float *__restrict__ out, float zscale) {
  constexpr int kPer = 16 / sizeof(E);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T || tile_skipped(bits, t)) return;  // whole wavefronts
  const int64_t y = targets[t];
  if (y < 0 || y >= V) {
    if (lane == 0) out[t] = __builtin_nanf("");
    return;
  }
  const E *hr = h + t * H;
  const E *wr = W + y * H;
  float acc = 0.f;
  for (int64_t c = (int64_t)lane * kPer; c < H; c += 64 * kPer) {
    const uint4 x = *reinterpret_cast<const uint4 *>(hr + c);
    const uint4 w = *reinterpret_cast<const uint4 *>(wr + c);
    if constexpr (sizeof(E) == 1) {
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc = __builtin_fmaf(e4m3_to_f32((xs[k] >> (8 * b)) & 0xffu), e4m3_to_f32((ws[k] >> (8 * b)) & 0xffu), acc);
    } else if constexpr (sizeof(E) == 2) {
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc = __builtin_fmaf(__uint_as_float(xs[k] << 16), __uint_as_float(ws[k] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(xs[k] & 0xffff0000u), __uint_as_float(ws[k] & 0xffff0000u), acc);
      }
    } else {
      acc = __builtin_fmaf(__uint_as_float(x.x), __uint_as_float(w.x), acc);
      acc = __builtin_fmaf(__uint_as_float(x.y), __uint_as_float(w.y), acc);
      acc = __builtin_fmaf(__uint_as_float(x.z), __uint_as_float(w.z), acc);
      acc = __builtin_fmaf(__uint_as_float(x.w), __uint_as_float(w.w), acc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) out[t] = acc * zscale;
}

// covered: NULL (every token's row was accumulated), or the bitmap of tokens the
// active metadata covers; an active token outside it gets a NaN row.
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(int64_t T_, int64_t H, const float *__restrict__ acc,
                                                       const uint8_t *__restrict__ mask,
                                                       const uint32_t *__restrict__ covered,
                                                       T *__restrict__ dh, float scale) {
  constexpr int kPer = 16 / sizeof(T);
  const int64_t per_row = H / kPer;
  const int64_t n = T_ * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / per_row;
    const int64_t c = (idx - t * per_row) * kPer;
    const bool act = mask ? (mask[t] != 0) : true;
    if (act && covered && !((covered[t >> 5] >> (t & 31)) & 1u)) {
      // an active token the metadata does not cover: its accumulator row was never written
      if constexpr (sizeof(T) == 2)
        *reinterpret_cast<uint4 *>(dh + t * H + c) = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);
      else
        *reinterpret_cast<uint4 *>(dh + t * H + c) = make_uint4(0x7fc00000u, 0x7fc00000u, 0x7fc00000u, 0x7fc00000u);
      continue;
    }
    if constexpr (sizeof(T) == 2) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (act) {
        float4 x0 = *reinterpret_cast<const float4 *>(acc + t * H + c);
        float4 x1 = *reinterpret_cast<const float4 *>(acc + t * H + c + 4);
        x0 = make_float4(x0.x * scale, x0.y * scale, x0.z * scale, x0.w * scale);
        x1 = make_float4(x1.x * scale, x1.y * scale, x1.z * scale, x1.w * scale);
        // pairs rounded to bf16 (nearest, ties to even) by v_cvt_pk_bf16_f32
        auto rne2 = [](float lo, float hi) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
        };
        w[0] = rne2(x0.x, x0.y);
        w[1] = rne2(x0.z, x0.w);
        w[2] = rne2(x1.x, x1.y);
        w[3] = rne2(x1.z, x1.w);
      }
      *reinterpret_cast<uint4 *>(dh + t * H + c) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (act) {
        x = *reinterpret_cast<const float4 *>(acc + t * H + c);
        x = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
      }
      *reinterpret_cast<float4 *>(dh + t * H + c) = x;
    }
  }
}

}  // namespace

hipError_t launch_spans(const uint8_t *mask, int64_t T, int32_t max_gap, int32_t tile_m,
                        int64_t span_cap, int32_t *spans, int32_t *num_spans, uint32_t *tile_bits,
                        int32_t *active_count, hipStream_t st) {
  hipLaunchKernelGGL(spans_kernel, dim3(1), dim3(kBlock), 0, st, mask, T, max_gap, tile_m, span_cap,
                     spans, num_spans, tile_bits, active_count);
  return hipGetLastError();
}

hipError_t launch_lists(int64_t T, const uint32_t *tile_bits, const int32_t *spans,
                        const int32_t *num_spans, int64_t span_cap, int32_t *tile_list,
                        int32_t *counts, int32_t *span_tiles, int64_t span_tile_cap, hipStream_t st,
                        uint32_t *covered) {
  hipLaunchKernelGGL(lists_kernel, dim3(1), dim3(kBlock), 0, st, T, tile_bits, spans, num_spans,
                     span_cap, tile_list, counts, span_tiles, span_tile_cap, covered);
  return hipGetLastError();
}

hipError_t launch_target_logit(int dtype, int64_t T, int64_t H, int64_t V, const void *h, const void *W,
                               const int64_t *targets, float *logprob, hipStream_t st,
                               const uint32_t *skip_bits, float zscale) {
  const unsigned tl_blocks = (unsigned)((T + 3) / 4);
  if (dtype == 2)
    hipLaunchKernelGGL(target_logit_kernel<uint8_t>, dim3(tl_blocks), dim3(256), 0, st, T, H, V,
                       reinterpret_cast<const uint8_t *>(h), reinterpret_cast<const uint8_t *>(W), targets,
                       skip_bits, logprob, zscale);
  else if (dtype == 1)
    hipLaunchKernelGGL(target_logit_kernel<uint16_t>, dim3(tl_blocks), dim3(256), 0, st, T, H, V,
                       reinterpret_cast<const uint16_t *>(h), reinterpret_cast<const uint16_t *>(W),
                       targets, skip_bits, logprob, 1.f);
  else
    hipLaunchKernelGGL(target_logit_kernel<float>, dim3(tl_blocks), dim3(256), 0, st, T, H, V,
                       reinterpret_cast<const float *>(h), reinterpret_cast<const float *>(W), targets,
                       skip_bits, logprob, 1.f);
  return hipGetLastError();
}

hipError_t launch_combine(int64_t T, int64_t V, const float *part, float *logprob, float *entropy,
                          float *lse, hipStream_t st, const uint32_t *skip_bits) {
  const int64_t blocks = (T + 63) / 64;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(64 * kCombWaves), 0, st, T, V,
                     reinterpret_cast<const float4 *>(part), skip_bits, logprob, entropy, lse);
  return hipGetLastError();
}

hipError_t launch_finalize(int dtype, int64_t T, int64_t H, const float *acc, const uint8_t *mask,
                           const uint32_t *covered, void *dh, hipStream_t st, float scale) {
  const int64_t per = dtype == 1 ? 8 : 4;
  const int64_t n = T * (H / per);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (dtype == 1)
    hipLaunchKernelGGL(finalize_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, T, H, acc,
                       mask, covered, reinterpret_cast<uint16_t *>(dh), scale);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, T, H, acc,
                       mask, covered, reinterpret_cast<float *>(dh), scale);
  return hipGetLastError();
}

}  // namespace flh

// ---------------------------------------------------------------------------------
// Blocked transpose through LDS: rows of `in` ([R][C]) are taken in blocks of `block`
// rows; block b becomes out_b = out + b * C * ld_out, [C][ld_out], with
// out_b[c][r] = in[b * block + r][c] and zeros in the padding columns past the
// block's rows.  A workgroup moves 64 x 64 tiles with 16-byte loads and stores,
// walking the tile grid with a stride of the launch size.  The backward uses it to
// lay W (one block per vocabulary split) and h out with the contraction index
// contiguous for the hidden- and weight-gradient products.
// Gather form (row_tiles set, one block): output column r takes input row
// row_tiles[r / 128] * 128 + r % 128 for r < 128 * n_row_tiles[0] (zero past R); the
// columns past that are not written.
namespace flh {
namespace {

constexpr int kTrTile = 64;

// Element conversion on the way through the tile: identity, or an E4M3 code to the
// bfloat16 pattern of its value (exact: every E4M3 value has at most 4 significant bits
// and an exponent inside bf16's range).
template <typename Ein, typename Eout>
__device__ __forceinline__ Eout tr_convert(Ein x) {
  if constexpr (sizeof(Ein) == 1)
    return (Eout)(__float_as_uint(e4m3_to_f32(x)) >> 16);
  else
    return x;
}

template <typename Ein, typename Eout>
__global__ __launch_bounds__(256) void transpose_kernel(const Ein *__restrict__ in, int64_t R, int64_t C,
                                                        Eout *__restrict__ out, int64_t ld_out, int64_t block,
                                                        int64_t c_tiles, int64_t r_tiles, int64_t n_tiles,
                                                        const int32_t *__restrict__ row_tiles,
                                                        const int32_t *__restrict__ n_row_tiles) {
  constexpr int kT = kTrTile;
  constexpr int kVi = 16 / sizeof(Ein);   // input elements per 16-byte vector
  constexpr int kVo = 16 / sizeof(Eout);  // output elements per 16-byte vector
  constexpr int kVecRowIn = kT / kVi;     // input vectors per tile row
  constexpr int kVecRowOut = kT / kVo;    // output vectors per tile column
  __shared__ Eout tile[kT][kT + kVo];     // padded rows
  const int tid = threadIdx.x;
  const bool gather = row_tiles != nullptr;
  const int64_t R_gather = gather ? (int64_t)n_row_tiles[0] * 128 : 0;
  for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    // tile (blk, rt, ct): rows blk * block + rt * 64 .., columns ct * 64 ..
    const int64_t blk = t / (r_tiles * c_tiles);
    const int64_t rem = t - blk * r_tiles * c_tiles;
    const int64_t rb = (rem / c_tiles) * kT, c0 = (rem % c_tiles) * kT;  // block-local row
    const int64_t r0 = blk * block + rb;                                   // row of `in`
    const int64_t R_blk = gather ? R_gather : ((R - blk * block) < block ? (R - blk * block) : block);
    if (gather && rb >= R_blk) continue;  // past the gathered rows: not written (whole workgroup)
    Eout *outb = out + blk * C * ld_out;
    for (int idx = tid; idx < kT * kVecRowIn; idx += 256) {
      const int rr = idx / kVecRowIn, cv = (idx % kVecRowIn) * kVi;
      const int64_t c = c0 + cv;
      int64_t r = r0 + rr;
      bool live = rb + rr < R_blk;  // a row of this block (rows past it read as 0)
      if (gather && live) {
        r = (int64_t)row_tiles[(rb + rr) >> 7] * 128 + ((rb + rr) & 127);
        live = r < R;
      }
      Ein v[kVi];
      if (live && c + kVi <= C) {
        const uint4 x = *reinterpret_cast<const uint4 *>(in + r * C + c);
        __builtin_memcpy(v, &x, 16);
      } else {
#pragma unroll
        for (int e = 0; e < kVi; ++e) v[e] = (live && c + e < C) ? in[r * C + c + e] : Ein(0);
      }
#pragma unroll
      for (int e = 0; e < kVi; ++e) tile[rr][cv + e] = tr_convert<Ein, Eout>(v[e]);
    }
    __syncthreads();
    for (int idx = tid; idx < kT * kVecRowOut; idx += 256) {
      const int cc = idx / kVecRowOut, rv = (idx % kVecRowOut) * kVo;
      const int64_t c = c0 + cc, r = rb + rv;  // block-local output column
      if (c >= C || r >= ld_out) continue;
      Eout v[kVo];
#pragma unroll
      for (int e = 0; e < kVo; ++e) v[e] = (r + e < R_blk) ? tile[rv + e][cc] : Eout(0);
      if (r + kVo <= ld_out) {
        uint4 x;
        __builtin_memcpy(&x, v, 16);
        *reinterpret_cast<uint4 *>(outb + c * ld_out + r) = x;
      } else {
        for (int e = 0; e < kVo && r + e < ld_out; ++e) outb[c * ld_out + r + e] = v[e];
      }
    }
    __syncthreads();  // the tile is refilled by the next iteration
  }
}

}  // namespace

hipError_t launch_transpose(int esz, const void *in, int64_t R, int64_t C, void *out, int64_t ld_out,
                            int64_t block, hipStream_t st, const int32_t *row_tiles,
                            const int32_t *n_row_tiles) {
  if (block <= 0) block = R;
  if (row_tiles && (block != R || !n_row_tiles)) return hipErrorInvalidValue;
  if (block % kTrTile != 0 && block != R) return hipErrorInvalidValue;
  const int64_t c_tiles = (C + kTrTile - 1) / kTrTile;
  const int64_t r_tiles = (ld_out + kTrTile - 1) / kTrTile;  // per block
  const int64_t n_blocks = (R + block - 1) / block;
  const int64_t n_tiles = n_blocks * r_tiles * c_tiles;
  if (n_tiles <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(n_tiles < (1 << 20) ? n_tiles : (1 << 20));
  if (esz == 1)
    hipLaunchKernelGGL((transpose_kernel<uint8_t, uint16_t>), dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint8_t *>(in), R, C, reinterpret_cast<uint16_t *>(out),
                       ld_out, block, c_tiles, r_tiles, n_tiles, row_tiles, n_row_tiles);
  else if (esz == 2)
    hipLaunchKernelGGL((transpose_kernel<uint16_t, uint16_t>), dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t *>(in), R, C, reinterpret_cast<uint16_t *>(out),
                       ld_out, block, c_tiles, r_tiles, n_tiles, row_tiles, n_row_tiles);
  else
    hipLaunchKernelGGL((transpose_kernel<float, float>), dim3(grid), dim3(256), 0, st,
                       reinterpret_cast<const float *>(in), R, C, reinterpret_cast<float *>(out), ld_out,
                       block, c_tiles, r_tiles, n_tiles, row_tiles, n_row_tiles);
  return hipGetLastError();
}

}  // namespace flh
