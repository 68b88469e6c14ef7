/*
 * f8lin.h -- C ABI of libf8lin.so, the MI355X (gfx950) Float8Linear library:
 * forward and backward of a linear layer Y = X W^T whose three GEMMs run in
 * fp8 with tensorwise scaling.
 *
 * What the library computes, with where it comes from:
 *  - Tensorwise dynamic scaling: one scale per tensor, from that tensor's
 *    current absolute maximum (amax), computed on the fly (pytorch/torchtitan
 *    PR #778 "Integrate float8nocompile", Summary).  The amax is computed by
 *    one of two algorithms that the PR's single-linear-layer benchmark table
 *    compares as kernel_algo ATOMIC_MAX and REDUCTION.
 *  - Delayed scaling of input, weight and grad_output: the scale comes from
 *    an amax history of past steps, updated after backward
 *    (pytorch/ao issue #1297, repro script: Float8LinearConfig with
 *    ScalingType.DELAYED, and sync_float8_amax_and_scale_history after
 *    loss.backward()).
 *  - The measured unit is the forward + backward of one linear layer
 *    (PR #778, "Benchmarking single linear layer forward+backward").
 * The arithmetic itself is not written on those pages; this library fixes
 * it as follows (the same definitions the tests check bit for bit):
 *    amax  = max_i |x_i|                   (exact; 0 for an empty tensor)
 *    scale = fmax / max(amax, 1e-12)       (IEEE binary32, correctly rounded)
 *    q     = RNE_sat(fl32(x * scale))      (binary32 multiply, then clamp to
 *                                           +-fmax, then round to nearest even
 *                                           onto the OCP fp8 grid; -0 stays -0;
 *                                           subnormals kept; NaN -> a NaN code)
 *    fmax  = 448 for OCP E4M3 (X, W), 57344 for OCP E5M2 (dY)
 *    Y  = (X8 W8^T)  / (s_x  s_w)   bf16, fp32 accumulation
 *    dX = (dY8 W8)   / (s_dy s_w)   bf16
 *    dW = (dY8^T X8) / (s_dy s_x)   bf16
 *
 * Conventions for every entry point:
 *  - Every data pointer is a DEVICE pointer owned by the caller, 16-byte
 *    aligned, to a row-major contiguous tensor.  bf16 tensors are passed as
 *    their uint16_t bit patterns; fp8 tensors as uint8_t codes.  A data
 *    pointer may be NULL only if its tensor has no elements.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it: nothing synchronises, nothing is read back to the
 *    host, nothing is allocated, and no pointer is kept after the call.
 *  - Matrix dimensions (rows, cols, M, N, K) must be >= 0, at most 2^22
 *    and multiples of 16 (every row is then a whole number of 16-byte
 *    vectors in both the row-major and the transposed layout).  A zero dimension is allowed and
 *    computes the degenerate result (e.g. dW = 0 when M = 0).
 *  - A transposed fp8 copy (qt of a (rows, cols) tensor; x8t (K, M), w8t
 *    (K, N), dy8t (N, M)) has cols rows of f8lin_transposed_ld(rows) bytes:
 *    the first `rows` bytes of each hold the codes, the rest (128 bytes, only
 *    when rows is a multiple of 32768) is padding the library never reads
 *    or writes.  Allocate cols * f8lin_transposed_ld(rows) bytes.
 *  - Arguments are checked before anything is launched; on error nothing is
 *    enqueued and a non-zero f8lin_status is returned.  F8LIN_EHIP reports a
 *    failed launch (hipGetLastError); faults during execution surface at the
 *    caller's next synchronisation.  Data-dependent conditions (NaN, Inf)
 *    are not errors.
 *  - Calls that share a workspace or a scaling state must be ordered (same
 *    stream, or synchronised).  The library keeps no global mutable state,
 *    except the per-device static scratch of f8lin_backward_noalloc.
 */
#ifndef F8LIN_H_
#define F8LIN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  F8LIN_OK = 0,
  F8LIN_EINVAL = 1,     /* null pointer, bad enum, overlapping buffers, bad count */
  F8LIN_ESHAPE = 2,     /* negative dimension, above 2^22, or not a multiple of 16 */
  F8LIN_EALIGN = 3,     /* a pointer not 16-byte aligned */
  F8LIN_EWORKSPACE = 4, /* workspace missing or smaller than f8lin_workspace_bytes() */
  F8LIN_EHIP = 5        /* a HIP launch failed */
} f8lin_status;

typedef enum { F8LIN_E4M3 = 0, F8LIN_E5M2 = 1 } f8lin_fmt;

/* The two amax algorithms of the single-linear benchmark (PR #778 table):
 * ATOMIC: every workgroup reduces its share and folds it with an atomic
 *         max into one of eight group slots; the last workgroup of a group
 *         folds the group into the tensor's slot, and the last group
 *         publishes the amax (one launch, no fences).
 * TWOPASS: every workgroup writes its partial max; a second pass reduces
 *          the partials: a one-workgroup launch in f8lin_amax, the cast
 *          kernel's prologue in f8lin_forward / f8lin_backward. */
typedef enum { F8LIN_AMAX_ATOMIC = 0, F8LIN_AMAX_TWOPASS = 1 } f8lin_amax_algo;

/* DYNAMIC: the scale comes from the tensor's current amax in state->amax:
 *          for f8lin_cast_transpose written beforehand by f8lin_amax; for
 *          f8lin_forward / f8lin_backward computed by the call itself (or
 *          handed in, with x_amax_given / dy_amax_given).
 * DELAYED: the scale comes from max(state->history[0..15]) (past steps only),
 *          and the cast also folds this tensor's amax into state->amax
 *          (which must hold 0 or a smaller value: f8lin_delayed_update resets
 *          it).  A role's first step has no history; callers run it in
 *          DYNAMIC mode (amax initialisation) and then call
 *          f8lin_delayed_update, which records it. */
typedef enum { F8LIN_DYNAMIC = 0, F8LIN_DELAYED = 1 } f8lin_scaling;

#define F8LIN_HISTORY_LEN 16

/* Scaling state of one tensor role (input, weight or grad_output); all
 * device pointers, caller-owned, zero-initialised before first use. */
typedef struct {
  float *amax;        /* [1] amax of the tensor (dynamic: written by f8lin_amax;
                         delayed: this step's amax, accumulated by the cast) */
  float *scale;       /* [2] written by the cast: {scale, 1/scale} */
  float *history;     /* [16] delayed only (may be NULL in dynamic mode) */
  int32_t *hist_meta; /* [2] delayed only: {count (0..16), pos (0..15)} */
} f8lin_state;

/* Bytes of device workspace that f8lin_amax / f8lin_forward /
 * f8lin_backward need.  A constant: the amax grid is capped at one
 * workgroup per compute unit, so no tensor size needs more (the scratch of
 * both amax algorithms of pytorch/torchtitan PR #778's single-linear-layer
 * table, ATOMIC_MAX and REDUCTION, plus the backward GEMM's work queue).
 * The caller zero-fills it once before first use.  Every call leaves the words that must start at zero (the
 * atomic algorithm's running maxima and tickets, the backward GEMM's
 * work-queue counters) at zero again; f8lin_amax
 * leaves the whole workspace zero-filled, while f8lin_forward /
 * f8lin_backward with the two-pass algorithm leave its partial maxima in
 * the workspace (every call overwrites them before reading them). */
size_t f8lin_workspace_bytes(void);

/* Row stride in bytes of the transposed fp8 copy of a tensor with `rows`
 * rows (each row of the copy holds `rows` codes): rows, or rows + 128 when
 * rows is a multiple of 32768 (GEMMs contracting along rows whose stride is
 * a multiple of 32 KB ran ~17% slower on MI355X: 4096 x 4096 x 65536 at a
 * 65536-byte stride 975-1032 us, at 65664 bytes 818-839 us).  0 for
 * rows < 0. */
int64_t f8lin_transposed_ld(int64_t rows);

/* Human-readable name of a status code (static string, never NULL; an
 * unknown code gives "unknown f8lin status"). */
const char *f8lin_status_str(int status);

/* amax of a bf16 tensor of n elements -> amax_out[0] (fp32): the tensorwise
 * absolute maximum that dynamic scaling takes its scale from
 * (pytorch/torchtitan PR #778, Summary, and its single-linear-layer table's
 * kernel_algo column: ATOMIC_MAX = F8LIN_AMAX_ATOMIC, REDUCTION =
 * F8LIN_AMAX_TWOPASS).  The result is exact (it is one of the inputs'
 * magnitudes), the same for both algorithms and for every launch order; NaN
 * inputs make it NaN; n = 0 gives 0.  x: n bf16 values, 16-byte aligned.
 * algo: f8lin_amax_algo.  ws: workspace of >= f8lin_workspace_bytes().
 * Errors: EINVAL (null amax_out, bad algo, output overlapping x), ESHAPE
 * (n < 0 or above 2^40), EALIGN, EWORKSPACE. */
int f8lin_amax(const uint16_t *x, int64_t n, int algo, float *amax_out, void *ws, size_t ws_bytes,
               void *stream);

/* Scale and cast of a bf16 (rows, cols) tensor to fp8 codes q (rows, cols),
 * and, if qt != NULL, the transposed copy qt (cols, rows), in one pass: the
 * "fp8 conversion" step that float8nocompile writes as handwritten kernels
 * (pytorch/torchtitan PR #778, Summary), with the scale taken as in
 * tensorwise dynamic or delayed scaling (pytorch/ao issue #1297, repro
 * script, CastConfig(ScalingType.DELAYED)).  The transposed copy is the
 * operand layout the backward GEMMs contract over.
 * fmt: f8lin_fmt.  mode: f8lin_scaling (see above).  The scale and inverse
 * scale the cast used are stored to st->scale[0..1]; in delayed mode this
 * tensor's amax is also folded into st->amax.
 * Errors: EINVAL (null state or state fields, bad enum, outputs overlapping
 * inputs), ESHAPE, EALIGN; nothing is launched on error. */
int f8lin_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, int fmt, int mode,
                         const f8lin_state *st, uint8_t *q, uint8_t *qt, void *stream);

/* The conversion alone, on fp32 values (scale 1): q[i] = RNE_sat(v[i]), the
 * rounding step of the cast above (for checking the conversion on every
 * binary32 input).  v: n fp32 values; q: n codes; both 16-byte aligned.
 * Errors: EINVAL, ESHAPE, EALIGN. */
int f8lin_cast_f32(const float *v, int64_t n, int fmt, uint8_t *q, void *stream);

/* fp8 GEMM with a per-tensor dequantisation epilogue, the product every
 * GEMM of the layer's forward + backward is an instance of (pytorch/torchtitan
 * PR #778, "Benchmarking single linear layer forward+backward
 * performance"):
 *   C (M, N) bf16 = (A (M, K) . B (N, K)^T) * inv_scale_a[0] * inv_scale_b[0]
 * A and B are fp8 codes in formats fmt_a / fmt_b, both contiguous along K;
 * products are exact and accumulate in fp32; the result is rounded once to
 * bf16 (nearest even) after the scaling.  K = 0 gives C = 0. */
int f8lin_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N, int64_t K,
               const float *inv_scale_a, const float *inv_scale_b, uint16_t *c, void *stream);

/* Several of those GEMMs in one launch (the backward runs its dgrad and
 * wgrad this way, pytorch/torchtitan PR #778, "Benchmarking single linear
 * layer forward+backward performance": both backward products of the
 * layer).  d[i] describes GEMM i exactly as the arguments of f8lin_gemm do;
 * all of them share the operand formats fmt_a / fmt_b.  count: 1 ..
 * F8LIN_MAX_BATCH.  Each C is computed as f8lin_gemm would (bit for bit).
 * Errors: as f8lin_gemm for each entry; an output overlapping any other
 * entry's input or output is F8LIN_EINVAL; nothing is launched unless every
 * entry is valid. */
#define F8LIN_MAX_BATCH 4
typedef struct {
  const uint8_t *a, *b;                      /* (M, K), (N, K) fp8 codes, K-contiguous */
  const float *inv_scale_a, *inv_scale_b;    /* [1] each */
  uint16_t *c;                               /* (M, N) bf16 output */
  int64_t M, N, K;
  int64_t lda, ldb; /* row strides of a and b in bytes: 0 (= K), or K <= ld <= 2^22 + 128, a multiple of 16
                       (e.g. a transposed copy's f8lin_transposed_ld) */
} f8lin_gemm_desc;
int f8lin_gemm_batch(const f8lin_gemm_desc *d, int count, int fmt_a, int fmt_b, void *stream);

/* Forward of the layer (pytorch/torchtitan PR #778, "Benchmarking single
 * linear layer forward+backward performance", the forward half):
 * X (M, K) bf16, W (N, K) bf16 -> Y (M, N) bf16.
 * Per tensor: amax (dynamic mode only), then one cast writing both layouts
 * (the transposed ones with the f8lin_transposed_ld row stride);
 * then Y = X8 . W8^T with the dequantisation epilogue.  x8t and w8t (and the
 * scales in sx, sw) are what backward needs; x8 and w8 can be reused or
 * freed after the call.
 * bias: optional (N) bf16 vector added to every row of Y in fp32 before the
 * rounding to bf16 (the linear layers of pytorch/ao issue #1297's repro
 * script keep nn.Linear's default bias); NULL for none.  16-byte aligned. */
typedef struct {
  int64_t M, N, K;
  const uint16_t *x, *w; /* inputs */
  uint16_t *y;           /* output (M, N) */
  uint8_t *x8, *x8t;     /* (M, K) e4m3 and its transpose (K, M) */
  uint8_t *w8, *w8t;     /* (N, K) e4m3 and its transpose (K, N) */
  f8lin_state sx, sw;
  int mode_x, mode_w; /* f8lin_scaling */
  int algo;           /* f8lin_amax_algo, for the dynamic-mode amax passes */
  void *ws;
  size_t ws_bytes;
  const uint16_t *bias; /* (N) bf16, or NULL */
  /* Nonzero: w8, w8t and sw.scale already hold the cast of this W from an
   * earlier forward (the weight is unchanged, e.g. between the micro-batches
   * of one optimizer step), so W's amax and cast are skipped and w is not
   * read. */
  int w_cast_valid;
  /* Optional (NULL = none) hipEvent_t handles, recorded on `stream` right
   * before and right after the call's GEMM launch: the duration of the
   * GEMM the call itself issues, for profiling. */
  void *ev_gemm_begin, *ev_gemm_end;
  /* Optional (NULL = none), 4-byte aligned: receives max |Y| over the bf16
   * values of Y (the amax of Y, exact, as f8lin_amax would give it), taken
   * in the GEMM's epilogue.  Handing it to the next layer as its sx.amax
   * with x_amax_given spares that layer its amax pass over Y: the float8
   * ops fused with the op that produces their input (pytorch/ao issue
   * #1199, the reply on the ops not being fused with surrounding ops). */
  float *y_amax;
  /* Nonzero (dynamic mode only): sx.amax already holds amax(X) -- e.g. the
   * y_amax of the layer that produced X -- so X's amax pass is skipped. */
  int x_amax_given;
} f8lin_fwd_args;

/* Backward of the layer (pytorch/torchtitan PR #778, "Benchmarking single
 * linear layer forward+backward performance", the backward half), given
 * dY (M, N) bf16 and the forward's saved x8t,
 * w8t and scaling states: dY is cast once to e5m2 (both layouts), then
 * dX (M, K) = dY8 . W8 (contraction over N, B operand w8t) and
 * dW (N, K) = dY8^T . X8 (contraction over M, A operand dy8t, B operand x8t),
 * each with its dequantisation epilogue.
 * dbias: optional (N) bf16 output, the bias gradient db[n] = sum over m of
 * dY[m, n] (from the bf16 dY, summed in fp32 in a fixed order -- the same
 * bits on every run -- and rounded once to bf16); NULL for none.  It needs
 * dbias_ws, a scratch buffer of >= f8lin_dbias_workspace_bytes(M, N) bytes
 * for the per-tile column sums (contents need no initialisation).  Both
 * 16-byte aligned.
 * gemm_ws: optional (NULL = none) scratch for GEMMs split along their
 * contraction: a GEMM with few 256x256 output tiles and a long contraction
 * (typically dW of a small weight over many tokens) leaves most CUs idle, so
 * with room in gemm_ws (f8lin_backward_gemm_workspace_bytes(M, N, K) bytes;
 * contents need no initialisation; 16-byte aligned) it runs as up to eight
 * K ranges whose fp32 partial products a second kernel sums in range order
 * (the same bits on every run), scales and rounds to bf16.  The summation
 * order differs from the unsplit GEMM's, so the results may differ from it
 * in the last bits, within the GEMM tolerance.
 * ws: required in dynamic mode (the amax); optional in delayed mode.  A
 * valid workspace (either mode) also holds the work-queue counters through
 * which dgrad and wgrad share their launch when their contraction lengths
 * differ; without one (delayed mode, ws NULL) they share it with a fixed
 * tile order -- the same results, bit for bit. */
typedef struct {
  int64_t M, N, K;
  const uint16_t *dy;           /* input (M, N) */
  const uint8_t *x8t, *w8t;     /* saved by forward: (K, M), (K, N) */
  uint16_t *dx, *dw;            /* outputs (M, K), (N, K) */
  uint8_t *dy8, *dy8t;          /* (M, N) e5m2 and its transpose (N, M) */
  f8lin_state sx, sw, sdy;      /* sx, sw: the forward's states (scales read) */
  int mode_dy;                  /* f8lin_scaling */
  int algo;                     /* f8lin_amax_algo */
  void *ws;
  size_t ws_bytes;
  uint16_t *dbias;              /* (N) bf16 output, or NULL */
  float *dbias_ws;              /* scratch for dbias, or NULL */
  size_t dbias_ws_bytes;
  void *gemm_ws;                /* scratch for split GEMMs, or NULL */
  size_t gemm_ws_bytes;
  void *ev_gemm_begin, *ev_gemm_end; /* as in f8lin_fwd_args (around the dgrad + wgrad launch) */
  float *dx_amax;               /* optional: receives amax(dX), as y_amax does amax(Y) */
  int dy_amax_given;            /* nonzero (dynamic mode only): sdy.amax holds amax(dY) */
} f8lin_bwd_args;

/* Bytes of dbias_ws that f8lin_backward needs for an (M, N) dY, for the
 * gradient of the bias the repro's nn.Linear layers keep (pytorch/ao issue
 * #1297, repro script): max(1, ceil(M / 128)) * N * 4.  0 for M or N < 0. */
size_t f8lin_dbias_workspace_bytes(int64_t M, int64_t N);

/* Bytes of gemm_ws with which f8lin_backward splits every GEMM of an
 * (M, N, K) layer that it would split (the backward GEMMs of pytorch/
 * torchtitan PR #778's single-linear-layer benchmark; 0: none is split at
 * this shape; also 0 for invalid dimensions).  With less, GEMMs whose
 * partials do not fit run unsplit. */
size_t f8lin_backward_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* The forward described above f8lin_fwd_args.  Errors, all checked before
 * anything is launched: EINVAL (null args or required pointers, bad enums,
 * a delayed state without history, x_amax_given outside dynamic mode,
 * any output overlapping another output or an input), ESHAPE, EALIGN,
 * EWORKSPACE (a dynamic-mode amax pass without a valid workspace); EHIP if
 * a launch fails. */
int f8lin_forward(const f8lin_fwd_args *args, void *stream);

/* Forward of count (1 .. F8LIN_MAX_BATCH) linears that read the same input X,
 * such as the q, k and v projections of an attention block or the two input
 * projections of a gated MLP (the Llama3 8b layer of pytorch/torchtitan
 * PR #778's training table has both): X is cast once (amax, scale, X8, X8^T), each
 * weight as in f8lin_forward, and the count GEMMs run in one launch.  Every
 * entry gives the same M, K, x, x8, x8t, sx, mode_x, algo and workspace;
 * N, w, y, w8, w8t, sw, mode_w, bias, w_cast_valid and y_amax are per
 * entry, and ev_gemm_begin / ev_gemm_end and x_amax_given are shared.  Each
 * output equals, bit for bit, what f8lin_forward gives for that entry.
 * Errors: as f8lin_forward for each entry; entries that disagree on the
 * shared fields, or outputs that overlap any entry's input or output, are
 * F8LIN_EINVAL; nothing is launched unless every entry is valid. */
int f8lin_forward_shared_x(const f8lin_fwd_args *args, int count, void *stream);

/* The backward described above f8lin_bwd_args.  Errors, all checked before
 * anything is launched: EINVAL (null args or required pointers, bad enums,
 * dy_amax_given outside dynamic mode, overlapping buffers -- the split
 * scratch counts for the part that split GEMMs would use), ESHAPE, EALIGN,
 * EWORKSPACE (dynamic mode without a valid workspace, a bias gradient
 * without enough dbias_ws); EHIP if a launch fails. */
int f8lin_backward(const f8lin_bwd_args *args, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * backward of f8lin_backward with no workspace from the caller.  args->ws,
 * args->dbias_ws and args->gemm_ws must be NULL; the library's own static
 * device scratch on the current device (8 KB of workspace words plus one
 * 16 MiB region, held by every GPU the library runs on until the process
 * ends) takes their place: the bias gradient's column sums and the split
 * GEMMs' partials share the region (GEMMs whose partials do not fit run
 * unsplit, as with a gemm_ws of 16 MiB).  `stream` must belong to the
 * current device.  Outputs equal, bit for bit, those of f8lin_backward
 * given a zeroed workspace, a dbias_ws and a 16 MiB gemm_ws.  Every call on
 * one GPU shares that scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race; order them.  The first call on a device
 * looks the scratch up and clears its workspace words with a kernel on
 * `stream`; no call allocates.
 * Errors: as f8lin_backward; also EINVAL if ws, dbias_ws or gemm_ws is
 * given, and EWORKSPACE if the bias gradient's column sums
 * (f8lin_dbias_workspace_bytes(M, N)) exceed 16 MiB. */
int f8lin_backward_noalloc(const f8lin_bwd_args *args, void *stream);

/* After backward, the sync step of delayed scaling
 * (pytorch/ao issue #1297, repro script: sync_float8_amax_and_scale_history
 * after loss.backward()), for each of the n_states states:
 *   history[pos] = amax; pos = (pos + 1) % 16; count = min(count + 1, 16);
 *   amax = 0.
 * Every state needs amax, history (16-byte aligned) and hist_meta.
 * A state's {count, pos} must be one those pushes reach from the zeroed
 * state: 0 <= count <= 16, 0 <= pos <= 15, and pos == count while
 * count < 16.  The host cannot see device memory, so this is checked on the
 * device: a state that fails it (e.g. restored from a corrupted checkpoint)
 * is left untouched -- history, meta and amax -- and, if status is not
 * NULL, status[i] (a device int32 array of n_states, 4-byte aligned) is set
 * to F8LIN_EINVAL for it and to F8LIN_OK for every state updated.
 * Errors (host-side, before any launch): EINVAL (null states, a state
 * without amax / history / hist_meta, n_states < 0, status overlapping a
 * state), EALIGN. */
int f8lin_delayed_update(const f8lin_state *states, int n_states, int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* F8LIN_H_ */
