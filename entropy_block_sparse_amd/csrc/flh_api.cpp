// Host side of the C ABI in include/flh.h: argument validation, workspace
// carve-up and the launch sequence of each call.  No device memory is allocated
// here and nothing waits on the device; every check happens before the first
// launch, so a rejected call enqueues nothing.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <vector>

#include "flh.h"
#include "flh_internal.h"

using namespace flh;

namespace {

constexpr int32_t kDefaultSplit = 16384;
// T, H, V < 2^24: a wave addresses its 64 rows of an operand from one buffer base with
// 32-bit byte offsets (row * row stride + stage offset), and the backward's transposed
// operands (h^T, the vocabulary-major d-logits staging) have rows of about T elements,
// so 64 rows of them stay within 2^32 bytes only for T well below 2^25.
constexpr int64_t kMaxDim = (int64_t)1 << 24;

enum KernelId : int32_t {
  kIdSpans = 0,
  kIdFwdGemm,
  kIdFwdCombine,
  kIdBwdLists,
  kIdDlogits,
  kIdDhidden,
  kIdDweight,
  kIdFinalize,
  kIdTranspose,
  kIdFwdLists,
  kIdFwdTarget,
  kIdCount
};
const char *const kKernelNames[kIdCount] = {
    "spans_build", "fwd_logits_softmax", "fwd_combine", "bwd_lists",
    "dlogits",     "dhidden_spans",      "dweight",     "dhidden_finalize",
    "transpose",   "fwd_lists",          "fwd_target_logit"};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
int64_t elt_size(flh_dtype dt) { return dt == FLH_BF16 ? 2 : (dt == FLH_FP8_E4M3 ? 1 : 4); }
// element of the d-logits staging and of the transposed copies: bf16 for fp8 inputs
int64_t stage_esz(flh_dtype dt) { return dt == FLH_F32 ? 4 : 2; }
bool dtype_ok(flh_dtype dt) { return dt == FLH_BF16 || dt == FLH_F32 || dt == FLH_FP8_E4M3; }

// How a call's contractions run: the launch dtype of the products over H (forward,
// d-logits), that of the hidden- and weight-gradient products over the bf16 or fp32
// staging, and the scales of fp8 inputs.
struct Prec {
  int kdt;        // 0 fp32, 1 bf16, 2 fp8 E4M3
  int stage_kdt;  // 0 fp32, 1 bf16
  float zscale;   // logits = zscale * accumulated products
  float scale_h;  // dW = scale_h * (D^T widened h codes)
  float scale_w;  // dH = scale_w * (D widened W codes)
};
Prec prec_of(flh_dtype dt, float scale_h = 1.f, float scale_w = 1.f) {
  if (dt == FLH_FP8_E4M3) return Prec{2, 1, scale_h * scale_w, scale_h, scale_w};
  return Prec{dt == FLH_BF16 ? 1 : 0, dt == FLH_BF16 ? 1 : 0, 1.f, 1.f, 1.f};
}
// fp8 scales: finite and positive, with a product (the logit scale) in [1e-30, 1e30] and small
// enough that no logit can leave the fp32 range: a logit is that product times a sum of H
// code products, each at most 448^2 in magnitude, accumulated in fp32.
bool scales_ok(float scale_h, float scale_w, int64_t H) {
  auto fin_pos = [](float x) { return x > 0.f && x <= 3.0e38f; };
  if (!fin_pos(scale_h) || !fin_pos(scale_w)) return false;
  const double z = (double)scale_h * (double)scale_w;
  if (!(z >= 1e-30 && z <= 1e30)) return false;
  return z * 448.0 * 448.0 * (double)(H > 0 ? H : 0) < 0x1p127;
}

// Sizes shared by both calls: T, H, V in [1, 2^24); H a multiple of one
// 16-byte chunk.
bool dims_ok(flh_dtype dt, int64_t T, int64_t H, int64_t V) {
  const int64_t per = 16 / elt_size(dt);
  return T > 0 && T < kMaxDim && V > 0 && V < kMaxDim && H > 0 && H < kMaxDim && H % per == 0;
}

int32_t split_or_default(int32_t s) { return s == 0 ? kDefaultSplit : s; }

// Row stride (elements) for a workspace matrix with n columns: a multiple of 64
// elements that is odd, so consecutive rows start an odd number of 128-byte lines
// apart (bf16) and the rows a load instruction touches spread over the memory
// channels instead of repeating one power-of-two stride.
int64_t pad_ld(int64_t n) {
  int64_t ld = cdiv(n, 64) * 64;
  if ((ld / 64) % 2 == 0) ld += 64;
  return ld;
}

// Forward workspace: per-tile softmax states [ceil(V/256)][T] float4, then (used by
// the forward over active token tiles only) counts and the token-tile list.
size_t fwd_part_bytes(int64_t T, int64_t V) { return (size_t)cdiv(V, kTile) * (size_t)T * 16; }
size_t fwd_counts_off(int64_t T, int64_t V) { return align_up(fwd_part_bytes(T, V), 256); }
size_t fwd_list_off(int64_t T, int64_t V) { return fwd_counts_off(T, V) + 256; }
size_t fwd_bytes(int64_t T, int64_t V) {
  return align_up(fwd_list_off(T, V) + (size_t)cdiv(T, kSkipTile) * sizeof(int32_t), 256);
}

struct BwdLayout {
  size_t counts, tile_list, span_tiles, covered, D, Dt, Wt, ht, acc, total;
  int64_t span_tile_cap, ld_wt, ld_t;
};

// Backward workspace: [counts | token-tile list | span-tile list | covered-token bits | d-logits
// staging [T][ld] sized by the widest live split | the same transposed, [W][ld_t] |
// W^T per split [splits][H][ld_wt] | h^T [H][ld_t] | fp32 dH accumulator].  The transposed copies put
// the contraction index of the hidden- and weight-gradient products in contiguous
// memory, so every contraction streams K-contiguous rows.
BwdLayout bwd_layout(flh_dtype dt, int64_t T, int64_t H, int64_t V, int32_t S) {
  BwdLayout L{};
  const int64_t n_skip = cdiv(T, kSkipTile);
  // span pieces: every span holds >= 1 token and spans are >= 1 token apart, so there
  // are <= ceil(T/2) spans and <= T/kSpanPiece + (number of spans) pieces
  L.span_tile_cap = cdiv(T, kSpanPiece) + (T + 1) / 2 + 1;
  const int64_t w_max = V < S ? V : S;
  const int64_t ld_max = pad_ld(w_max);
  L.ld_wt = pad_ld(w_max);
  L.ld_t = pad_ld(cdiv(T, kSkipTile) * kSkipTile);  // room for whole 128-token tiles
  const size_t esz = (size_t)stage_esz(dt);
  size_t off = 0;
  L.counts = off;
  off = align_up(off + 64, 256);
  L.tile_list = off;
  off = align_up(off + (size_t)n_skip * 4, 256);
  L.span_tiles = off;
  off = align_up(off + (size_t)L.span_tile_cap * 8, 256);
  L.covered = off;
  off = align_up(off + (size_t)cdiv(T, 32) * 4, 256);
  L.D = off;
  off = align_up(off + (size_t)T * (size_t)ld_max * esz, 256);
  L.Dt = off;
  off = align_up(off + (size_t)w_max * (size_t)L.ld_t * esz, 256);
  L.Wt = off;
  off = align_up(off + (size_t)cdiv(V, S) * (size_t)H * (size_t)L.ld_wt * esz, 256);
  L.ht = off;
  off = align_up(off + (size_t)H * (size_t)L.ld_t * esz, 256);
  L.acc = off;
  off = align_up(off + (size_t)T * (size_t)H * 4, 256);
  L.total = off;
  return L;
}

int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int grid_for(int64_t upper_items, int cus) {
  int64_t g = upper_items < cus ? upper_items : cus;
  return g < 1 ? 1 : (int)g;
}

// ---- launch tracing (per host thread) ----
struct Trace {
  bool on = false;
  int32_t cap = 0, n = 0;
  std::vector<hipEvent_t> ev;
  std::vector<int32_t> kid, split;
};
Trace &trace() {
  thread_local Trace tr;
  return tr;
}

template <class F>
flh_status run(int32_t kid, int32_t split, hipStream_t st, F &&f) {
  Trace &tr = trace();
  const bool rec = tr.on && tr.n < tr.cap;
  if (rec && hipEventRecord(tr.ev[2 * tr.n], st) != hipSuccess) return FLH_E_HIP;
  if (f() != hipSuccess) return FLH_E_HIP;
  if (rec) {
    if (hipEventRecord(tr.ev[2 * tr.n + 1], st) != hipSuccess) return FLH_E_HIP;
    tr.kid[tr.n] = kid;
    tr.split[tr.n] = split;
    ++tr.n;
  }
  return FLH_OK;
}

}  // namespace

namespace {
flh_status forward_run(const Prec &pr, flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                       int64_t T, int64_t H, int64_t V, float *logprob, float *entropy, float *lse,
                       const flh_active_meta *meta, void *ws, size_t ws_bytes, void *stream, uint32_t flags);
flh_status backward_run(const Prec &pr, flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                        const float *lse, const float *entropy, const float *grad_logprob,
                        const float *grad_entropy, const uint8_t *loss_mask, const flh_active_meta *meta,
                        int64_t T, int64_t H, int64_t V, int32_t vocab_split, void *d_hidden, void *d_weight,
                        void *ws, size_t ws_bytes, void *stream, uint32_t flags);
}  // namespace

// Every check of a forward call except those of the workspace.
flh_status flh::forward_check(flh_dtype dt, const void *h, const void *W, const int64_t *targets, int64_t T,
                              int64_t H, int64_t V, const float *logprob, const float *entropy,
                              const float *lse, const flh_active_meta *meta, uint32_t flags) {
  if (!dtype_ok(dt)) return FLH_E_DTYPE;
  if (flags & ~(uint32_t)FLH_FWD_SKIP_INACTIVE) return FLH_E_UNSUPPORTED;
  if (!h || !W || !targets || !logprob || !entropy || !lse) return FLH_E_NULL;
  if (!dims_ok(dt, T, H, V)) return FLH_E_SHAPE;
  if (flags & FLH_FWD_SKIP_INACTIVE) {
    if (!meta) return FLH_E_META;
    if (!meta->tile_bits) return FLH_E_NULL;
    if (meta->T != T || meta->tile_m != flh_tile_m(dt)) return FLH_E_META;
  }
  if (!aligned(h, 16) || !aligned(W, 16)) return FLH_E_ALIGN;
  return FLH_OK;
}

extern "C" {

int32_t flh_abi_version(void) { return FLH_ABI_VERSION; }

const char *flh_status_string(flh_status s) {
  switch (s) {
    case FLH_OK: return "ok";
    case FLH_E_NULL: return "a required pointer is NULL";
    case FLH_E_SHAPE: return "invalid size";
    case FLH_E_DTYPE: return "unknown dtype";
    case FLH_E_ALIGN: return "misaligned pointer";
    case FLH_E_WORKSPACE: return "workspace too small";
    case FLH_E_META: return "active metadata inconsistent with the call";
    case FLH_E_UNSUPPORTED: return "unsupported request";
    case FLH_E_HIP: return "HIP runtime error";
    case FLH_E_SCRATCH: return "sizes exceed the library's static scratch (flh_forward_noalloc)";
    case FLH_E_SCALE: return "an fp8 scale is not finite and positive, or their product leaves [1e-30, 1e30]";
  }
  return "unknown status";
}

int32_t flh_tile_m(flh_dtype dt) { return dtype_ok(dt) ? kSkipTile : 0; }

int64_t flh_span_capacity(int64_t T, int32_t max_gap) {
  if (T <= 0 || max_gap < 0) return 0;
  return (T + (int64_t)max_gap + 1) / ((int64_t)max_gap + 2);
}

size_t flh_workspace_bytes(flh_op op, flh_dtype dt, int64_t T, int64_t H, int64_t V,
                           int32_t vocab_split) {
  if (!dtype_ok(dt)) return 0;
  switch (op) {
    case FLH_OP_SPANS: return 0;
    case FLH_OP_FORWARD: return dims_ok(dt, T, H, V) ? fwd_bytes(T, V) : 0;
    case FLH_OP_BACKWARD: {
      const int32_t S = split_or_default(vocab_split);
      if (!dims_ok(dt, T, H, V) || S <= 0 || S % kTile != 0) return 0;
      return bwd_layout(dt, T, H, V, S).total;
    }
  }
  return 0;
}

flh_status flh_spans_build(const uint8_t *loss_mask, flh_active_meta *meta, void *ws,
                           size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (!loss_mask || !meta) return FLH_E_NULL;
  if (!meta->spans || !meta->num_spans || !meta->tile_bits || !meta->active_count) return FLH_E_NULL;
  if (meta->T <= 0 || meta->T >= kMaxDim || meta->tile_m <= 0) return FLH_E_SHAPE;
  if (meta->max_gap < 0) return FLH_E_META;
  if (meta->span_cap < flh_span_capacity(meta->T, meta->max_gap)) return FLH_E_META;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return run(kIdSpans, -1, st, [&] {
    return launch_spans(loss_mask, meta->T, meta->max_gap, meta->tile_m, meta->span_cap,
                        meta->spans, meta->num_spans, meta->tile_bits, meta->active_count, st);
  });
}

flh_status flh_forward(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                       int64_t T, int64_t H, int64_t V, float *logprob, float *entropy, float *lse,
                       void *ws, size_t ws_bytes, void *stream) {
  return flh_forward_ex(dt, h, W, targets, T, H, V, logprob, entropy, lse, nullptr, ws, ws_bytes, stream, 0u);
}

flh_status flh_forward_ex(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                          int64_t T, int64_t H, int64_t V, float *logprob, float *entropy, float *lse,
                          const flh_active_meta *meta, void *ws, size_t ws_bytes, void *stream,
                          uint32_t flags) {
  if (dt == FLH_FP8_E4M3) return FLH_E_UNSUPPORTED;  // fp8 inputs need their scales: flh_forward_fp8
  return forward_run(prec_of(dt), dt, h, W, targets, T, H, V, logprob, entropy, lse, meta, ws, ws_bytes, stream,
                     flags);
}

flh_status flh_forward_fp8(const uint8_t *h, float scale_h, const uint8_t *W, float scale_w,
                           const int64_t *targets, int64_t T, int64_t H, int64_t V, float *logprob,
                           float *entropy, float *lse, const flh_active_meta *meta, void *ws, size_t ws_bytes,
                           void *stream, uint32_t flags) {
  if (!scales_ok(scale_h, scale_w, H)) return FLH_E_SCALE;
  return forward_run(prec_of(FLH_FP8_E4M3, scale_h, scale_w), FLH_FP8_E4M3, h, W, targets, T, H, V, logprob,
                     entropy, lse, meta, ws, ws_bytes, stream, flags);
}

}  // extern "C"

namespace {

flh_status forward_run(const Prec &pr, flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                       int64_t T, int64_t H, int64_t V, float *logprob, float *entropy, float *lse,
                       const flh_active_meta *meta, void *ws, size_t ws_bytes, void *stream, uint32_t flags) {
  const flh_status chk = flh::forward_check(dt, h, W, targets, T, H, V, logprob, entropy, lse, meta, flags);
  if (chk != FLH_OK) return chk;
  const bool skip = (flags & FLH_FWD_SKIP_INACTIVE) != 0;
  if (!ws) return FLH_E_NULL;
  if (!aligned(ws, 256)) return FLH_E_ALIGN;
  if (ws_bytes < fwd_bytes(T, V)) return FLH_E_WORKSPACE;
  const int cus = num_cus();
  if (cus <= 0) return FLH_E_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  GemmArgs a{};
  a.T = T;
  a.H = H;
  a.V = V;
  a.h = h;
  a.W = W;
  a.targets = targets;
  a.part = reinterpret_cast<float *>(ws);
  a.zscale = pr.zscale;
  a.out_scale = 1.f;
  flh_status s = FLH_OK;
  if (skip) {
    // the active token tiles, ascending (the list builder without span pieces)
    char *base = reinterpret_cast<char *>(ws);
    a.counts = reinterpret_cast<int32_t *>(base + fwd_counts_off(T, V));
    a.tile_list = reinterpret_cast<int32_t *>(base + fwd_list_off(T, V));
    a.n_skip_tiles = (int32_t)cdiv(T, kSkipTile);
    s = run(kIdFwdLists, -1, st, [&] {
      return launch_lists(T, meta->tile_bits, nullptr, nullptr, 0, const_cast<int32_t *>(a.tile_list),
                          const_cast<int32_t *>(a.counts), nullptr, 0, st);
    });
    if (s != FLH_OK) return s;
    const int grid = grid_for(cdiv(V, kTile) * cdiv(a.n_skip_tiles, 2), cus);
    s = run(kIdFwdGemm, -1, st, [&] { return launch_gemm(pr.kdt, kFwdSkip, a, grid, st); });
  } else {
    const int grid = grid_for(cdiv(V, kTile) * cdiv(T, kTile), cus);
    s = run(kIdFwdGemm, -1, st, [&] { return launch_gemm(pr.kdt, kFwd, a, grid, st); });
  }
  if (s != FLH_OK) return s;
  const uint32_t *skip_bits = skip ? meta->tile_bits : nullptr;
  s = run(kIdFwdTarget, -1, st, [&] {
    return launch_target_logit(pr.kdt, T, H, V, h, W, targets, logprob, st, skip_bits, pr.zscale);
  });
  if (s != FLH_OK) return s;
  return run(kIdFwdCombine, -1, st, [&] {
    return launch_combine(T, V, a.part, logprob, entropy, lse, st, skip_bits);
  });
}

}  // namespace

extern "C" {

flh_status flh_backward(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                        const float *lse, const float *entropy, const float *grad_logprob,
                        const float *grad_entropy, const uint8_t *loss_mask,
                        const flh_active_meta *meta, int64_t T, int64_t H, int64_t V,
                        int32_t vocab_split, void *d_hidden, void *d_weight, void *ws,
                        size_t ws_bytes, void *stream) {
  return flh_backward_ex(dt, h, W, targets, lse, entropy, grad_logprob, grad_entropy, loss_mask, meta, T,
                         H, V, vocab_split, d_hidden, d_weight, ws, ws_bytes, stream, 0u);
}

flh_status flh_backward_ex(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                           const float *lse, const float *entropy, const float *grad_logprob,
                           const float *grad_entropy, const uint8_t *loss_mask,
                           const flh_active_meta *meta, int64_t T, int64_t H, int64_t V,
                           int32_t vocab_split, void *d_hidden, void *d_weight, void *ws,
                           size_t ws_bytes, void *stream, uint32_t flags) {
  if (dt == FLH_FP8_E4M3) return FLH_E_UNSUPPORTED;  // fp8 inputs need their scales: flh_backward_fp8
  return backward_run(prec_of(dt), dt, h, W, targets, lse, entropy, grad_logprob, grad_entropy, loss_mask, meta,
                      T, H, V, vocab_split, d_hidden, d_weight, ws, ws_bytes, stream, flags);
}

flh_status flh_backward_fp8(const uint8_t *h, float scale_h, const uint8_t *W, float scale_w,
                            const int64_t *targets, const float *lse, const float *entropy,
                            const float *grad_logprob, const float *grad_entropy, const uint8_t *loss_mask,
                            const flh_active_meta *meta, int64_t T, int64_t H, int64_t V, int32_t vocab_split,
                            void *d_hidden, void *d_weight, void *ws, size_t ws_bytes, void *stream,
                            uint32_t flags) {
  if (!scales_ok(scale_h, scale_w, H)) return FLH_E_SCALE;
  return backward_run(prec_of(FLH_FP8_E4M3, scale_h, scale_w), FLH_FP8_E4M3, h, W, targets, lse, entropy,
                      grad_logprob, grad_entropy, loss_mask, meta, T, H, V, vocab_split, d_hidden, d_weight, ws,
                      ws_bytes, stream, flags);
}

}  // extern "C"

namespace {

flh_status backward_run(const Prec &pr, flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                        const float *lse, const float *entropy, const float *grad_logprob,
                        const float *grad_entropy, const uint8_t *loss_mask, const flh_active_meta *meta,
                        int64_t T, int64_t H, int64_t V, int32_t vocab_split, void *d_hidden, void *d_weight,
                        void *ws, size_t ws_bytes, void *stream, uint32_t flags) {
  if (!dtype_ok(dt)) return FLH_E_DTYPE;
  if (flags & ~(uint32_t)(FLH_BWD_SKIP_INACTIVE_DW | FLH_BWD_PADDED_TAIL)) return FLH_E_UNSUPPORTED;
  // the padded probe computes tiles with no live vocabulary row, which the fp32 load
  // path cannot address (it clamps onto the last live row)
  if ((flags & FLH_BWD_PADDED_TAIL) && dt == FLH_F32) return FLH_E_UNSUPPORTED;
  if (!h || !W || !targets || !lse || !entropy || !d_hidden || !d_weight || !ws) return FLH_E_NULL;
  const int32_t S = split_or_default(vocab_split);
  if (!dims_ok(dt, T, H, V) || S <= 0 || S % kTile != 0) return FLH_E_SHAPE;
  if (meta) {
    if (!loss_mask) return FLH_E_META;
    if (!meta->spans || !meta->num_spans || !meta->tile_bits) return FLH_E_NULL;
    // the span list must be able to hold every span this mask can have, as in
    // flh_spans_build: a smaller capacity would have dropped spans
    if (meta->T != T || meta->tile_m != flh_tile_m(dt) || meta->max_gap < 0 ||
        meta->span_cap < flh_span_capacity(T, meta->max_gap))
      return FLH_E_META;
  }
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(d_hidden, 16) || !aligned(d_weight, 16) ||
      !aligned(ws, 256))
    return FLH_E_ALIGN;
  const BwdLayout L = bwd_layout(dt, T, H, V, S);
  if (ws_bytes < L.total) return FLH_E_WORKSPACE;
  const int cus = num_cus();
  if (cus <= 0) return FLH_E_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char *base = reinterpret_cast<char *>(ws);

  GemmArgs a{};
  a.T = T;
  a.H = H;
  a.V = V;
  a.h = h;
  a.W = W;
  a.targets = targets;
  a.lse = lse;
  a.entropy = entropy;
  a.grad_lp = grad_logprob;
  a.grad_ent = grad_entropy;
  a.mask = loss_mask;
  a.counts = reinterpret_cast<int32_t *>(base + L.counts);
  a.tile_list = reinterpret_cast<int32_t *>(base + L.tile_list);
  a.span_tiles = reinterpret_cast<int32_t *>(base + L.span_tiles);
  a.n_skip_tiles = (int32_t)cdiv(T, kSkipTile);
  a.D = base + L.D;
  a.Dt = base + L.Dt;
  a.Wt = base + L.Wt;
  a.ht = base + L.ht;
  a.ld_wt = L.ld_wt;
  a.ld_t = L.ld_t;
  a.dh_acc = reinterpret_cast<float *>(base + L.acc);
  a.dW = d_weight;
  a.zscale = pr.zscale;
  a.out_scale = 1.f;
  // without metadata every tile is active and the compact layout is the dense one
  a.compact_dw = (flags & FLH_BWD_SKIP_INACTIVE_DW) && meta ? 1 : 0;

  flh_status s = run(kIdBwdLists, -1, st, [&] {
    return launch_lists(T, meta ? meta->tile_bits : nullptr, meta ? meta->spans : nullptr,
                        meta ? meta->num_spans : nullptr, meta ? meta->span_cap : 0,
                        reinterpret_cast<int32_t *>(base + L.tile_list),
                        reinterpret_cast<int32_t *>(base + L.counts),
                        reinterpret_cast<int32_t *>(base + L.span_tiles), L.span_tile_cap, st,
                        meta ? reinterpret_cast<uint32_t *>(base + L.covered) : nullptr);
  });
  if (s != FLH_OK) return s;
  // (fp8 codes are widened to bf16 on the way: the transposed copies feed bf16 products)
  s = run(kIdTranspose, -1, st, [&] {
    return launch_transpose((int)elt_size(dt), W, V, H, base + L.Wt, L.ld_wt, S, st);
  });
  if (s != FLH_OK) return s;
  s = run(kIdTranspose, -1, st, [&] {
    if (a.compact_dw)  // h^T over the active token tiles only, in tile-list order
      return launch_transpose((int)elt_size(dt), h, T, H, base + L.ht, L.ld_t, 0, st, a.tile_list, a.counts);
    return launch_transpose((int)elt_size(dt), h, T, H, base + L.ht, L.ld_t, 0, st);
  });
  if (s != FLH_OK) return s;

  const int64_t n_splits = cdiv(V, S);
  const int64_t h_tiles = cdiv(H, kTile);
  for (int64_t sp = 0; sp < n_splits; ++sp) {
    // live width of this split: the staging row stride and every grid below
    // come from it, never from S.
    const int64_t Ws = (V - sp * S) < S ? (V - sp * S) : S;
    const int64_t ld_prev = a.ld_d;
    a.v_base = sp * S;
    a.Ws = (int32_t)Ws;
    a.Ws_grid = (flags & FLH_BWD_PADDED_TAIL) ? (V < S ? V : S) : Ws;
    a.ld_d = (int32_t)pad_ld(a.Ws_grid);
    a.first_split = sp == 0;
    // inactive token tiles: zero staging once per layout (the first split is the widest)
    a.zero_vm = sp == 0 && !a.compact_dw;
    a.zero_tm = sp == 0 || a.ld_d != ld_prev;
    a.Wt = base + L.Wt + (size_t)sp * (size_t)H * (size_t)L.ld_wt * (size_t)stage_esz(dt);
    const int32_t tag = (int32_t)sp;
    const int64_t v_tiles = cdiv(a.Ws_grid, kTile);
    s = run(kIdDlogits, tag, st, [&] {
      return launch_gemm(pr.kdt, kDlogits, a, grid_for(v_tiles * cdiv(a.n_skip_tiles, 2), cus), st);
    });
    if (s != FLH_OK) return s;
    s = run(kIdDhidden, tag, st, [&] {
      return launch_gemm(pr.stage_kdt, kDhidden, a,
                         grid_for(cdiv(L.span_tile_cap, kPiecesPerTile) * h_tiles, cus), st);
    });
    if (s != FLH_OK) return s;
    s = run(kIdDweight, tag, st, [&] {
      GemmArgs aw = a;
      aw.out_scale = pr.scale_h;
      return launch_gemm(pr.stage_kdt, pr.kdt == 2 ? kDweightS : kDweight, aw, grid_for(v_tiles * h_tiles, cus),
                         st);
    });
    if (s != FLH_OK) return s;
  }
  return run(kIdFinalize, -1, st, [&] {
    return launch_finalize(pr.stage_kdt, T, H, a.dh_acc, loss_mask,
                           meta ? reinterpret_cast<const uint32_t *>(base + L.covered) : nullptr, d_hidden, st,
                           pr.scale_w);
  });
}

}  // namespace

extern "C" {

flh_status flh_trace_begin(int32_t capacity) {
  Trace &tr = trace();
  if (tr.on || capacity <= 0) return FLH_E_UNSUPPORTED;
  tr.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto &e : tr.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto &x : tr.ev)
        if (x) (void)hipEventDestroy(x);
      tr.ev.clear();
      return FLH_E_HIP;
    }
  tr.kid.assign(capacity, -1);
  tr.split.assign(capacity, -1);
  tr.cap = capacity;
  tr.n = 0;
  tr.on = true;
  return FLH_OK;
}

int32_t flh_trace_end(flh_trace_record *records, int32_t max_records) {
  Trace &tr = trace();
  if (!tr.on) return -1;
  int32_t n = tr.n;
  bool err = false;
  for (int32_t i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(tr.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, tr.ev[2 * i], tr.ev[2 * i + 1]) != hipSuccess)
      err = true;
    if (records && i < max_records) records[i] = flh_trace_record{tr.kid[i], tr.split[i], ms};
  }
  for (auto &e : tr.ev) (void)hipEventDestroy(e);
  tr.ev.clear();
  tr.on = false;
  tr.n = 0;
  return err ? -1 : n;
}

const char *flh_kernel_name(int32_t kernel_id) {
  return (kernel_id >= 0 && kernel_id < kIdCount) ? kKernelNames[kernel_id] : "unknown";
}

}  // extern "C"
