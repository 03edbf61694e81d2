/*
 * flh.h -- C ABI of the block-sparse fused LM head for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described on the page "perf(megatron): add
 * block-sparse fused LM-head backward" (NovaSky-AI/SkyRL pull request 2376,
 * cited below as "SkyRL #2376" with the page's section headings):
 *
 *   forward   z = h W^T computed tile by tile, never stored as [T, V]; an online
 *             log-softmax gives each token's target log-prob and entropy
 *             ("What does this PR do?", Bugbot "Overview": fused linear log-prob;
 *             the stack's "fuse LM-head entropy for RL" layer).
 *   metadata  a forward active mask (here a tile bitmap) and ordered active spans,
 *             runs of the loss mask coalesced across gaps <= 128 tokens
 *             ("How it works"; Bugbot "Overview").
 *   backward  d-logits recomputed only for active token tiles; the hidden gradient
 *             accumulated span by span, split by split (Gemini "Code Review":
 *             d_hidden += split_d_logits @ split_weight); the final vocabulary
 *             split staged at its live width with every launch sized from that
 *             width (Greptile "Wide-tail grid exceeds live split"); the weight
 *             gradient a dense contraction over all tokens ("How it works").
 *
 * Definitions (fp32 accumulation; inputs bf16 or fp32):
 *   lse[t]     = log sum_v exp(z[t,v])
 *   logprob[t] = z[t, targets[t]] - lse[t]
 *   entropy[t] = sum_v p[t,v] (lse[t] - z[t,v]),  p = exp(z - lse)   (nats)
 *   ga = m * grad_logprob, gb = m * grad_entropy  (m = loss mask, NULL grad = 0)
 *   dz[t,v]    = ga[t] ([v == y_t] - p) + gb[t] p (lse[t] - entropy[t] - z[t,v])
 *   d_hidden   = dz W,  d_weight = dz^T h
 *
 * Conventions (every entry point):
 *   - All array arguments are DEVICE pointers into memory the caller owns; the
 *     library never allocates or frees device memory and keeps no per-call
 *     state.  Scratch memory is the caller's workspace (`ws`, `ws_bytes`), sized
 *     by flh_workspace_bytes() and at least 256-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is only enqueued: no host/device synchronisation, no device-to-host reads,
 *     so a whole forward+backward can be captured into a HIP graph.
 *   - Matrices are row-major and contiguous: h [T,H], W [V,H], d_hidden [T,H],
 *     d_weight [V,H].  h, W, d_hidden, d_weight must be 16-byte aligned and H a
 *     multiple of 16 bytes of elements (8 for bf16, 4 for fp32).
 *   - T, H and V are at most 2^24 - 1 (else FLH_E_SHAPE): the kernels address a
 *     wave's 64 operand rows from one base with 32-bit byte offsets, and the
 *     backward's transposed operands have rows about T elements long.
 *   - Every argument is checked on the host before anything is launched; a bad
 *     argument returns an error status and enqueues nothing.  FLH_E_HIP means a
 *     launch failed (its work may be partially enqueued).  Nothing aborts and no
 *     exception crosses the ABI.
 *   - Not checked (that would need a device read): targets in [0, V) (a target
 *     out of range gives logprob = NaN for that token), finite inputs, and that
 *     `meta` was built from the same loss mask.  flh_backward reads the metadata's
 *     spans clamped to [0, T] (and their count to span_cap), so metadata of another
 *     mask never sends a launch outside its buffers, and an active token that such
 *     metadata leaves out (outside every span, or in a tile whose bit is clear) gets a
 *     NaN d_hidden row rather than a silently wrong or zero one.
 *   - Results are bit-identical from run to run (no floating-point atomics).
 *   - Calls on different streams may run concurrently if their buffers differ.
 */
#ifndef FLH_H_
#define FLH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLH_ABI_VERSION 1

/* The enums below are int-sized in C; compiled as C++ they get `int` as their fixed
 * underlying type, so that any value a C caller passes (an unknown dtype, say) is a
 * valid value of the type and is rejected by the checks rather than being undefined. */
#ifdef __cplusplus
#define FLH_ENUM_INT : int
#else
#define FLH_ENUM_INT
#endif

typedef enum FLH_ENUM_INT {
  FLH_OK = 0,
  FLH_E_NULL = 1,        /* a required pointer is NULL                               */
  FLH_E_SHAPE = 2,       /* a size is <= 0, too large, or not a supported multiple   */
  FLH_E_DTYPE = 3,       /* unknown dtype                                            */
  FLH_E_ALIGN = 4,       /* a matrix pointer or the workspace is misaligned          */
  FLH_E_WORKSPACE = 5,   /* ws_bytes smaller than flh_workspace_bytes()              */
  FLH_E_META = 6,        /* active metadata inconsistent with this call              */
  FLH_E_UNSUPPORTED = 7, /* valid request the library does not support               */
  FLH_E_HIP = 8,         /* a HIP runtime call or kernel launch failed               */
  FLH_E_SCRATCH = 9,     /* sizes exceed the static scratch (flh_forward_noalloc)   */
  FLH_E_SCALE = 10       /* an fp8 scale is not usable (flh_forward_fp8/backward_fp8) */
} flh_status;

/* FLH_FP8_E4M3: OCP E4M3 codes (see flh_forward_fp8); accepted by the queries
 * (flh_tile_m, flh_workspace_bytes) and the fp8 entry points only. */
typedef enum FLH_ENUM_INT { FLH_F32 = 0, FLH_BF16 = 1, FLH_FP8_E4M3 = 2 } flh_dtype;

/* Which call a workspace size is for. */
typedef enum FLH_ENUM_INT { FLH_OP_SPANS = 0, FLH_OP_FORWARD = 1, FLH_OP_BACKWARD = 2 } flh_op;

/*
 * Active metadata derived from the loss mask (SkyRL #2376, "How it works": one
 * builder derives the forward active mask and the backward spans).  The struct
 * itself is host memory; every pointer in it is device memory owned by the
 * caller.  The caller fills T, max_gap, tile_m, span_cap and the four pointers;
 * flh_spans_build fills the arrays.
 *
 *   spans       [span_cap][2] int32, half-open (start, end) in flat packed token
 *               coordinates, ascending and disjoint.  A span starts and ends on an
 *               active token; two consecutive runs of active tokens share a span
 *               iff at most max_gap inactive tokens lie between them (Bugbot
 *               "Overview": gaps <= 128).  Sequence boundaries are not seen.
 *   num_spans   device int32 scalar: number of spans written.
 *   tile_bits   [ceil(ceil(T/tile_m)/32)] uint32; bit i%32 of word i/32 (least
 *               significant first) is set iff any token of
 *               [i*tile_m, min(T,(i+1)*tile_m)) is active.  Unused bits are 0.
 *   active_count device int32 scalar: number of active tokens A.
 */
typedef struct {
  int64_t T;            /* tokens the metadata describes                             */
  int32_t max_gap;      /* G >= 0 (the page uses 128)                                */
  int32_t tile_m;       /* bitmap tile height; flh_backward requires flh_tile_m(dt)  */
  int64_t span_cap;     /* capacity of `spans`, >= flh_span_capacity(T, max_gap)     */
  int32_t *spans;
  int32_t *num_spans;
  uint32_t *tile_bits;
  int32_t *active_count;
} flh_active_meta;

/* ABI version of the loaded library (FLH_ABI_VERSION it was built with). */
int32_t flh_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *flh_status_string(flh_status s);

/* Token-tile height of the d-logits tile skip: the tile_m flh_backward expects. */
int32_t flh_tile_m(flh_dtype dt);

/* Largest possible number of spans: floor((T + G + 1) / (G + 2)); 0 for T <= 0. */
int64_t flh_span_capacity(int64_t T, int32_t max_gap);

/*
 * Workspace bytes the call `op` needs for these sizes (0 for FLH_OP_SPANS).
 * vocab_split 0 means 16384.  Returns 0 for invalid sizes as well.
 * Forward: per-tile softmax partials, ceil(V/256) * T * 16 bytes, and the active
 * token-tile list (4 * ceil(T/128) bytes plus alignment).
 * Backward: work lists and a token bitmap; the d-logits staging of the widest split in two layouts
 * (token-major T x W and vocabulary-major W x T, W = min(V, vocab_split)); W and h
 * transposed (H x V and H x T, so that every contraction reads its contraction
 * index contiguously); and an fp32 T x H hidden-gradient accumulator.  For
 * T = 16384, H = 4096, V = 128256 in bf16 this is about 2.5 GB.
 */
size_t flh_workspace_bytes(flh_op op, flh_dtype dt, int64_t T, int64_t H, int64_t V,
                           int32_t vocab_split);

/*
 * Builds the active metadata from the loss mask on the device.
 *   loss_mask  [T] uint8, nonzero = active (the RL loss mask, Bugbot "Overview").
 *   meta       host struct, see flh_active_meta; meta->T is the length of the mask.
 * Errors: FLH_E_NULL (mask, meta or a meta pointer NULL), FLH_E_SHAPE (T <= 0 or
 * T >= 2^24, tile_m <= 0), FLH_E_META (max_gap < 0 or span_cap too small).
 */
flh_status flh_spans_build(const uint8_t *loss_mask, flh_active_meta *meta, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * Forward: per-token target log-prob, entropy and log-sum-exp, never storing the
 * [T, V] logits (SkyRL #2376, "What does this PR do?"; fused entropy layer).
 *   dt        FLH_BF16 or FLH_F32, the dtype of h and W.
 *   h [T,H], W [V,H], targets [T] int64 in [0, V).
 *   logprob, entropy, lse: [T] fp32 outputs (lse and entropy are what
 *   flh_backward needs saved).
 *   ws        at least flh_workspace_bytes(FLH_OP_FORWARD, dt, T, H, V, 0) bytes.
 */
flh_status flh_forward(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                       int64_t T, int64_t H, int64_t V, float *logprob, float *entropy,
                       float *lse, void *ws, size_t ws_bytes, void *stream);

/* Options of flh_forward_ex. */
enum {
  /* Forward over the active 128-token tiles only (the block-sparse forward of the
   * stack's previous layer, which the pages' baseline already includes; SkyRL #2376,
   * "Performance" and the stack listed under "What does this PR do?").  Tokens of a
   * tile without an active token get logprob = entropy = lse = 0; every other token's
   * outputs equal the dense forward's bitwise.  Needs meta (from flh_spans_build on the
   * loss mask), FLH_E_META without it or for a meta of another T or tile height. */
  FLH_FWD_SKIP_INACTIVE = 1u
};

/*
 * flh_forward with options: `flags` is a bitwise OR of FLH_FWD_* values (0 gives
 * flh_forward; meta is then ignored and may be NULL).  Arguments, workspace and errors
 * as for flh_forward, and FLH_E_UNSUPPORTED for an unknown flag bit.  A backward after
 * it is exact: inactive tokens' saved values are never read.
 */
flh_status flh_forward_ex(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                          int64_t T, int64_t H, int64_t V, float *logprob, float *entropy,
                          float *lse, const flh_active_meta *meta, void *ws, size_t ws_bytes,
                          void *stream, uint32_t flags);

/*
 * FP8 inputs.  The pages list FP8 among the layouts the span builder serves (SkyRL
 * #2376, Bugbot "Overview") and give no recipe; these calls take h and W as codes of
 * the OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; x1111111 is NaN; largest finite 448) with one fp32 scale per tensor:
 *   h[t,k] = scale_h * value(h[t,k]),   W[v,k] = scale_w * value(W[v,k]),
 * and compute on those values exactly what flh_forward_ex / flh_backward_ex compute
 * (definitions above).  The contractions over H (forward, d-logits) run on the codes
 * with fp8 matrix instructions and fp32 accumulation, the logits being the accumulated
 * products times scale_h * scale_w; the hidden- and weight-gradient products run in
 * bf16 on the codes widened exactly to bf16, with scale_w and scale_h applied to their
 * fp32 results.
 *   h [T,H], W [V,H]: uint8 codes, row-major, 16-byte aligned; H a multiple of 16.
 *   scale_h, scale_w: finite and > 0, with scale_h * scale_w in [1e-30, 1e30] and
 *   scale_h * scale_w * 448^2 * H < 2^127 (no logit, a sum of H code products of at most
 *   448^2 each times the scales, can leave the fp32 range), else FLH_E_SCALE.
 *   Workspace: flh_workspace_bytes(op, FLH_FP8_E4M3, ...).
 * flh_forward_fp8: arguments, options (FLH_FWD_*) and outputs as flh_forward_ex.
 */
flh_status flh_forward_fp8(const uint8_t *h, float scale_h, const uint8_t *W, float scale_w,
                           const int64_t *targets, int64_t T, int64_t H, int64_t V, float *logprob,
                           float *entropy, float *lse, const flh_active_meta *meta, void *ws,
                           size_t ws_bytes, void *stream, uint32_t flags);

/*
 * flh_forward_ex for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same call
 * without a workspace argument.  Its scratch (the per-tile softmax states and the
 * active-tile list) is a static device array of FLH_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU the library runs on, held until the process ends.  The call
 * allocates nothing (no hipMalloc, no library routine that allocates); its address is
 * looked up once per device, on the first call made with that device current.
 *   Limit: flh_workspace_bytes(FLH_OP_FORWARD, dt, T, H, V, 0) must not exceed
 *   FLH_NOALLOC_SCRATCH_BYTES (128 MiB: for V = 128256, up to T = 16743 tokens), else
 *   FLH_E_SCRATCH and nothing is enqueued.  Other arguments and errors as for
 *   flh_forward_ex (bf16 and fp32 inputs; FLH_FP8_E4M3: FLH_E_UNSUPPORTED).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (every byte a call reads was written earlier in the same call, so nothing
 *   needs clearing): calls that may overlap on one GPU (other streams, other host
 *   threads) race and must be serialised by the caller.
 */
#define FLH_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
flh_status flh_forward_noalloc(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                               int64_t T, int64_t H, int64_t V, float *logprob, float *entropy,
                               float *lse, const flh_active_meta *meta, void *stream, uint32_t flags);

/*
 * Backward: d_hidden [T,H] and d_weight [V,H] (dtype dt, both overwritten) from
 * the upstream gradients of logprob and entropy.
 *   lse, entropy   [T] fp32 as written by flh_forward for the same inputs.
 *   grad_logprob   [T] fp32 or NULL (zero).
 *   grad_entropy   [T] fp32 or NULL (zero: the no-grad entropy mode).
 *   loss_mask      [T] uint8 or NULL (all tokens active).  Gradients of inactive
 *                  tokens are ignored and their d_hidden rows are exactly +0.
 *   meta           NULL: dense fallback (every token tile computed, dense hidden
 *                  projection; SkyRL #2376 "Overview": the full dense projection
 *                  when no spans are provided).  Otherwise metadata built from
 *                  `loss_mask` by flh_spans_build: d-logits tiles without an active
 *                  token are skipped and d_hidden is projected over the spans only
 *                  ("How it works").  Requires loss_mask != NULL, meta->T == T,
 *                  meta->tile_m == flh_tile_m(dt), meta->max_gap >= 0 and
 *                  meta->span_cap >= flh_span_capacity(T, meta->max_gap), else
 *                  FLH_E_META (a smaller span list could have dropped spans, whose
 *                  tokens would then get no gradient: Bugbot "Note").
 *   vocab_split    split width S (0 = 16384), a multiple of 256.  Split s covers
 *                  vocabulary rows [s*S, s*S + W_s) with W_s = min(S, V - s*S); its
 *                  d-logits staging buffer and every launch over it are sized by
 *                  the live width W_s (SkyRL #2376, "How it works" and the Greptile
 *                  finding on the wide-tail grid).
 *   ws             at least flh_workspace_bytes(FLH_OP_BACKWARD, dt, T, H, V,
 *                  vocab_split) bytes.
 */
flh_status flh_backward(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                        const float *lse, const float *entropy, const float *grad_logprob,
                        const float *grad_entropy, const uint8_t *loss_mask,
                        const flh_active_meta *meta, int64_t T, int64_t H, int64_t V,
                        int32_t vocab_split, void *d_hidden, void *d_weight, void *ws,
                        size_t ws_bytes, void *stream);

/* Options of flh_backward_ex. */
enum {
  /* Weight gradient over the active token tiles only.  Rows of d-logits of tokens in
   * a tile without an active token are zero, so leaving those tiles out of
   * dW = D^T h changes no product: the result is the dense one (bitwise, since the
   * remaining partial sums are formed in the same groups and order).  The
   * vocabulary-major staging and h^T then hold only the active tiles, so no zeros
   * are stored or read for the others.  This is the next step the analysis of the
   * method lists after the dense weight gradient, which the pages keep dense on
   * purpose (SkyRL #2376, "How it works": weight gradients stay a dense
   * contraction).  Has no effect when meta is NULL (every tile is active). */
  FLH_BWD_SKIP_INACTIVE_DW = 1u,
  /* Measurement probe of the baseline that the live-width split replaces (SkyRL #2376,
   * "Performance": live-width final vocabulary split against padded staging): every
   * split, the last included, is staged and launched at the widest split's width
   * min(V, vocab_split), with the padding columns zero.  The results equal the default's
   * bitwise; only the time differs.  bf16 only (FLH_E_UNSUPPORTED for fp32). */
  FLH_BWD_PADDED_TAIL = 2u
};

/*
 * flh_backward with options: `flags` is a bitwise OR of FLH_BWD_* values (0 gives
 * flh_backward).  Arguments, workspace and errors as for flh_backward, and
 * FLH_E_UNSUPPORTED for an unknown flag bit.  (dt FLH_FP8_E4M3: flh_backward_fp8.)
 */
flh_status flh_backward_ex(flh_dtype dt, const void *h, const void *W, const int64_t *targets,
                           const float *lse, const float *entropy, const float *grad_logprob,
                           const float *grad_entropy, const uint8_t *loss_mask,
                           const flh_active_meta *meta, int64_t T, int64_t H, int64_t V,
                           int32_t vocab_split, void *d_hidden, void *d_weight, void *ws,
                           size_t ws_bytes, void *stream, uint32_t flags);

/*
 * Backward for FP8 inputs (see flh_forward_fp8): d_hidden [T,H] and d_weight [V,H] in
 * bf16 (gradients with respect to the dequantized h and W), from the lse and entropy
 * flh_forward_fp8 saved.  Other arguments, options (FLH_BWD_*) and errors as for
 * flh_backward_ex, plus FLH_E_SCALE.
 */
flh_status flh_backward_fp8(const uint8_t *h, float scale_h, const uint8_t *W, float scale_w,
                            const int64_t *targets, const float *lse, const float *entropy,
                            const float *grad_logprob, const float *grad_entropy,
                            const uint8_t *loss_mask, const flh_active_meta *meta, int64_t T,
                            int64_t H, int64_t V, int32_t vocab_split, void *d_hidden,
                            void *d_weight, void *ws, size_t ws_bytes, void *stream,
                            uint32_t flags);

/*
 * Launch tracing (profiling aid).  Between flh_trace_begin and flh_trace_end on
 * the same host thread, every kernel launch of the calls above is bracketed by a
 * pair of HIP events recorded on that call's stream (at most `capacity`
 * launches; later ones are not traced).  flh_trace_end waits for the events,
 * writes up to max_records records and returns how many launches were traced
 * (or -1 on a HIP error).  Tracing creates HIP events, so it is not for use
 * under graph capture.
 */
typedef struct {
  int32_t kernel_id;    /* see flh_kernel_name                                      */
  int32_t split;        /* vocabulary split index, -1 when not split-local          */
  float ms;             /* elapsed time between the two events                      */
} flh_trace_record;

flh_status flh_trace_begin(int32_t capacity);
int32_t flh_trace_end(flh_trace_record *records, int32_t max_records);
const char *flh_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* FLH_H_ */
