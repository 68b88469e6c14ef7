// Host-side launchers of the gfx950 kernels (one per kernel family), called by
// the C-ABI layer in api.hip after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/f8lin.h"

namespace f8lin {

// Row stride (bytes) of the transposed fp8 copy of a tensor with n rows: each
// of its rows holds n codes.  Strides that are multiples of 32 KB made the
// GEMMs that contract along such rows ~17% slower (a 4096 x 4096 x 65536
// product: 975-1032 us at a 65536-byte stride, 818-839 us at 65664), so
// those get 128 bytes of padding (never read or written).
constexpr int64_t kTransposeBadStride = 32768, kTransposePad = 128;
inline int64_t transposed_ld(int64_t n) { return (n > 0 && n % kTransposeBadStride == 0) ? n + kTransposePad : n; }

// Workspace layout (uint32 words): for tensor t of a launch, words
// [kWsSlotWords*t, +2) hold the atomic variant's running max and ticket;
// words [kWsPartialsOffset + kMaxGrid*t, +kMaxGrid) the two-pass partials;
// words [kWsGroupOffset + kWsSlotWords*(kAmaxGroups*t + g), +2) the atomic
// variant's group g running max and ticket (one 128-byte line each);
// words [kWsQueueOffset + kQueueWords*x, +2) the backward GEMM's work-queue
// counter and done ticket of XCD x (one line each).
constexpr int kMaxAmaxTensors = 2;
constexpr int kMaxGrid = 256;  // amax workgroups per tensor: one per CU
constexpr int kWsSlotWords = 32;
constexpr int kWsPartialsOffset = 64;
constexpr int kAmaxGroups = 8;
constexpr int kWsGroupOffset = kWsPartialsOffset + kMaxGrid * kMaxAmaxTensors;
constexpr int kQueueWords = 32;
constexpr int kWsQueueOffset = kWsGroupOffset + kWsSlotWords * kAmaxGroups * kMaxAmaxTensors;
constexpr size_t kWorkspaceBytes = 8192;
static_assert((kWsQueueOffset + kQueueWords * 8) * 4 <= (int)kWorkspaceBytes, "workspace layout");

struct AmaxTensor {
  const uint16_t *x;
  int64_t n;
  float *out;
};
hipError_t launch_amax(const AmaxTensor *ts, int count, int algo, uint32_t *ws, hipStream_t stream);
// The two-pass amax's first pass alone: tensor t's partial maxima (15-bit
// magnitudes) are left at parts[t][0 .. nparts[t]) inside the workspace, for
// the cast to reduce in its prologue (ts[t].out is not written).
hipError_t launch_amax_partials(const AmaxTensor *ts, int count, uint32_t *ws, const uint32_t **parts, int *nparts,
                                hipStream_t stream);

// Up to two casts (same format and scaling mode) in one launch.
struct CastTensor {
  const uint16_t *x;
  int64_t rows, cols;
  const f8lin_state *st;
  uint8_t *q, *qt;
  // dynamic mode: partial maxima of the two-pass amax to reduce (then
  // st->amax is written), or null to read st->amax
  const uint32_t *partials = nullptr;
  int npartials = 0;
  // dynamic mode, at most kSelfAmaxElems elements: the cast computes the
  // amax itself (every workgroup over the whole tensor; st->amax is written)
  int self_amax = 0;
  // if set (e5m2 only): fp32 column sums of x over each 128-row tile,
  // colsum[tile_row * cols + col], for the bias gradient
  float *colsum = nullptr;
  int64_t ldt = 0;  // row stride of qt in bytes (0: rows)
};
// Up to kMaxZero fp32 words the cast launch sets to +0 (from its first
// workgroup) before anything later on the stream runs: the output-amax words
// that the GEMM launch after it folds its results into.
constexpr int kMaxZero = 4;
struct ZeroWords {
  float *w[kMaxZero] = {nullptr, nullptr, nullptr, nullptr};
  int n = 0;
};
hipError_t launch_cast(const CastTensor *ts, int count, int fmt, int mode, hipStream_t stream,
                       const ZeroWords &zero = ZeroWords());

// Bias gradient: db[n] = bf16(sum over t < tiles of colsum[t * n_cols + n]),
// summed in order of t.
hipError_t launch_dbias(const float *colsum, int64_t tiles, int64_t n_cols, uint16_t *db, hipStream_t stream);
constexpr int kCastTile = 128;
// Tensors this small (128 Ki elements, 256 KB) have their amax computed inside
// the cast launch instead of by an amax launch of their own: at 16 x 4096 the
// separate launch cost ~3.5 us, more than every workgroup reading the whole
// 128 KB tensor from the L2.
constexpr int64_t kSelfAmaxElems = 128 * 1024;

hipError_t launch_cast_f32(const float *v, int64_t n, int fmt, uint8_t *q, hipStream_t stream);

hipError_t launch_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N,
                       int64_t K, const float *inv_a, const float *inv_b, uint16_t *c, hipStream_t stream);

// Up to kMaxGemms GEMMs with the same operand formats in one persistent
// launch (the backward's dgrad and wgrad; forwards sharing their input).
constexpr int kMaxGemms = 4;
struct GemmDesc {
  const uint8_t *a, *b;
  const float *inv_a, *inv_b;
  uint16_t *c;
  int64_t M, N, K;
  const uint16_t *bias = nullptr;  // (N) bf16 added to every row, or null
  // if set: max |C| over the rounded bf16 output is folded into *amax_out
  // (atomic max on the fp32 bit pattern; the word must hold +0 or less)
  float *amax_out = nullptr;
  int64_t lda = 0, ldb = 0;  // row strides of A and B in bytes (0: K)
};
// split_ws (optional, 16-byte aligned): room for the fp32 partial products of
// problems split along K (split_factor > 1); a problem that does not fit
// runs unsplit.  Contents need no initialisation.
// queue (optional): the workspace's work-queue words (zero; left zero), with
// which problems of different K share a launch through a work queue.
hipError_t launch_gemms(const GemmDesc *d, int count, int fmt_a, int fmt_b, hipStream_t stream,
                        void *split_ws = nullptr, size_t split_bytes = 0, uint32_t *queue = nullptr);
// K ranges a problem is split into when a partial-product workspace is given
// (1: not split), and the bytes its partials need.
int split_factor(int64_t M, int64_t N, int64_t K);
size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_delayed_update(const f8lin_state *states, int n, hipStream_t stream);

}  // namespace f8lin
