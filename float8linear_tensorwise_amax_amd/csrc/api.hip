// C ABI of libf8lin (declared in include/f8lin.h): argument validation, then
// the launch sequence of each entry point on the caller's stream.  Nothing
// here synchronises, reads device memory, or allocates.
//
// Forward / backward orchestration follows the layer's definition:
//   forward : [amax X, W] (one launch); cast X -> X8, X8^T and W -> W8, W8^T
//             (one launch when both tensors share a scaling mode);
//             Y = X8 . W8^T / (s_x s_w)
//   backward: [amax dY] cast dY -> dY8, dY8^T (e5m2);
//             dX = dY8 . (W8^T)^T / (s_dy s_w); dW = dY8^T . (X8^T)^T / (s_dy s_x)
// (amax passes only for tensors in dynamic mode; in delayed mode the cast
// takes its scale from the history and accumulates this step's amax.)
// The delayed-scaling history update runs after backward, as the sync call
// after loss.backward() does in pytorch/ao issue #1297's repro script.
#include <stdint.h>
#include <string.h>

#include <cstring>
#include <mutex>

#include "device_common.h"
#include "internal.h"

// Scratch of f8lin_backward_noalloc (see static_scratch below): the
// workspace words, then one 16 MiB region.
constexpr size_t kStaticRegionBytes = (size_t)16 << 20;
constexpr size_t kStaticScratchBytes = f8lin::kWorkspaceBytes + kStaticRegionBytes;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace f8lin {
namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 22;        // per matrix dimension (32-bit tile offsets)
constexpr int64_t kMaxElems = (int64_t)1 << 40;      // per tensor
constexpr int kUpdateBatch = 16;

struct StateBatch {
  f8lin_state s[kUpdateBatch];
  int n;
};

// A state is valid when it is one that pushes from the zeroed state can
// reach: 0 <= count <= 16, 0 <= pos < 16, and pos == count until the ring
// is full.  An invalid state (e.g. a corrupted checkpoint) is left as it is
// and reported in status[i] (F8LIN_EINVAL; F8LIN_OK otherwise) when the
// caller passes a status array.
__global__ void delayed_update_kernel(StateBatch batch, int32_t *status) {
  const int i = threadIdx.x;
  if (i >= batch.n) return;
  const f8lin_state st = batch.s[i];
  const int32_t count = st.hist_meta[0];
  const int32_t pos = st.hist_meta[1];
  const bool valid = count >= 0 && count <= kHistLen && pos >= 0 && pos < kHistLen && (count == kHistLen || pos == count);
  if (status) status[i] = valid ? F8LIN_OK : F8LIN_EINVAL;
  if (!valid) return;
  st.history[pos] = st.amax[0];
  st.hist_meta[1] = (pos + 1) % kHistLen;
  st.hist_meta[0] = count < kHistLen ? count + 1 : kHistLen;
  st.amax[0] = 0.0f;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// A data pointer may be NULL only when its tensor is empty.
bool missing(const void *p, int64_t elems) { return p == nullptr && elems > 0; }

bool bad_dim(int64_t d) { return d < 0 || d > kMaxDim || (d % 16) != 0; }

struct Range {
  const void *p;
  int64_t bytes;
};

bool overlaps(const Range &a, const Range &b) {
  if (a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + (uintptr_t)a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + (uintptr_t)b.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output range must be disjoint from every other range.
bool any_overlap(const Range *outs, int nout, const Range *ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return true;
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return true;
  }
  return false;
}

int check_fmt(int f) { return (f == F8LIN_E4M3 || f == F8LIN_E5M2) ? F8LIN_OK : F8LIN_EINVAL; }
int check_algo(int a) { return (a == F8LIN_AMAX_ATOMIC || a == F8LIN_AMAX_TWOPASS) ? F8LIN_OK : F8LIN_EINVAL; }
int check_mode(int m) { return (m == F8LIN_DYNAMIC || m == F8LIN_DELAYED) ? F8LIN_OK : F8LIN_EINVAL; }

int check_state(const f8lin_state &st, int mode) {
  if (!st.amax || !st.scale) return F8LIN_EINVAL;
  if (mode == F8LIN_DELAYED && (!st.history || !st.hist_meta)) return F8LIN_EINVAL;
  return F8LIN_OK;
}

int check_ws(const void *ws, size_t ws_bytes) {
  if (!ws || ws_bytes < kWorkspaceBytes || !aligned16(ws)) return F8LIN_EWORKSPACE;
  return F8LIN_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? F8LIN_OK : F8LIN_EHIP; }

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// Records an optional timing event on the call's stream.
int record(void *ev, hipStream_t s) {
  return ev ? status_of(hipEventRecord((hipEvent_t)ev, s)) : F8LIN_OK;
}

#define F8_TRY(expr)                 \
  do {                               \
    const int st_ = (expr);          \
    if (st_ != F8LIN_OK) return st_; \
  } while (0)

// Validation shared by f8lin_cast_transpose and the orchestrated casts.
int validate_cast(const uint16_t *x, int64_t rows, int64_t cols, int fmt, int mode, const f8lin_state *st,
                  const uint8_t *q, const uint8_t *qt) {
  if (!st) return F8LIN_EINVAL;
  F8_TRY(check_fmt(fmt));
  F8_TRY(check_mode(mode));
  F8_TRY(check_state(*st, mode));
  if (bad_dim(rows) || bad_dim(cols) || rows * cols > kMaxElems) return F8LIN_ESHAPE;
  if (missing(x, rows * cols) || missing(q, rows * cols)) return F8LIN_EINVAL;
  if (!aligned16(x) || !aligned16(q) || (qt && !aligned16(qt))) return F8LIN_EALIGN;
  const int64_t n = rows * cols;
  const Range outs[3] = {{q, n}, {qt, qt ? cols * transposed_ld(rows) : 0}, {st->scale, 8}};
  const Range ins[3] = {{x, 2 * n}, {st->amax, 4}, {st->history, mode == F8LIN_DELAYED ? 64 : 0}};
  if (any_overlap(outs, 3, ins, 3)) return F8LIN_EINVAL;
  return F8LIN_OK;
}

int validate_gemm(const uint8_t *a, int fa, const uint8_t *b, int fb, int64_t M, int64_t N, int64_t K,
                  const float *ia, const float *ib, const uint16_t *c, int64_t lda = 0, int64_t ldb = 0) {
  if (!ia || !ib) return F8LIN_EINVAL;
  F8_TRY(check_fmt(fa));
  F8_TRY(check_fmt(fb));
  if (bad_dim(M) || bad_dim(N) || bad_dim(K) || M * K > kMaxElems || N * K > kMaxElems || M * N > kMaxElems)
    return F8LIN_ESHAPE;
  if (lda == 0) lda = K;
  if (ldb == 0) ldb = K;
  // a row stride: at least K, a multiple of 16, at most kMaxDim + 128 (32-bit tile offsets)
  if (lda < K || ldb < K || lda % 16 || ldb % 16 || lda > kMaxDim + kTransposePad || ldb > kMaxDim + kTransposePad)
    return F8LIN_ESHAPE;
  if (missing(a, M * K) || missing(b, N * K) || missing(c, M * N)) return F8LIN_EINVAL;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return F8LIN_EALIGN;
  const Range outs[1] = {{c, 2 * M * N}};
  const Range ins[4] = {{a, M * lda}, {b, N * ldb}, {ia, 4}, {ib, 4}};
  if (any_overlap(outs, 1, ins, 4)) return F8LIN_EINVAL;
  return F8LIN_OK;
}

// Forward of `count` linears sharing X (count 1 is f8lin_forward): every
// argument is checked before anything is launched; then amax + cast of X and
// of each weight whose cast is not reused (two tensors of one scaling mode
// per launch, each two-pass amax launch directly followed by the cast that
// reduces its partials), then one GEMM launch for all of them.
int forward_impl(const f8lin_fwd_args *list, int count, void *stream) {
  if (!list || count < 1 || count > kMaxGemms) return F8LIN_EINVAL;
  const f8lin_fwd_args &a0 = list[0];
  F8_TRY(check_mode(a0.mode_x));
  F8_TRY(check_algo(a0.algo));
  F8_TRY(check_state(a0.sx, a0.mode_x));
  if (bad_dim(a0.M) || bad_dim(a0.K) || a0.M * a0.K > kMaxElems) return F8LIN_ESHAPE;
  const int64_t M = a0.M, K = a0.K, mk = M * K;
  if (missing(a0.x, mk) || missing(a0.x8, mk) || missing(a0.x8t, mk)) return F8LIN_EINVAL;
  if (!aligned16(a0.x) || !aligned16(a0.x8) || !aligned16(a0.x8t)) return F8LIN_EALIGN;
  // an amax of X handed in (from the producer's epilogue) replaces X's amax pass: dynamic mode only
  const bool x_given = a0.x_amax_given != 0;
  if (x_given && a0.mode_x != F8LIN_DYNAMIC) return F8LIN_EINVAL;
  bool need_ws = a0.mode_x == F8LIN_DYNAMIC && !x_given;
  Range outs[4 + 6 * kMaxGemms + 1], ins[2 + 6 * kMaxGemms];
  int no = 0, ni = 0;
  outs[no++] = {a0.x8, mk};
  outs[no++] = {a0.x8t, K * transposed_ld(M)};
  outs[no++] = {a0.sx.scale, 8};
  if (x_given)
    ins[ni++] = {a0.sx.amax, 4};
  else
    outs[no++] = {a0.sx.amax, 4};
  ins[ni++] = {a0.x, 2 * mk};
  ins[ni++] = {a0.sx.history, a0.mode_x == F8LIN_DELAYED ? 64 : 0};
  for (int i = 0; i < count; ++i) {
    const f8lin_fwd_args &a = list[i];
    if (i > 0 && (a.x != a0.x || a.x8 != a0.x8 || a.x8t != a0.x8t || a.M != M || a.K != K || a.mode_x != a0.mode_x ||
                  a.algo != a0.algo || a.ws != a0.ws || a.ws_bytes != a0.ws_bytes ||
                  a.x_amax_given != a0.x_amax_given || a.ev_gemm_begin != a0.ev_gemm_begin ||
                  a.ev_gemm_end != a0.ev_gemm_end || std::memcmp(&a.sx, &a0.sx, sizeof(f8lin_state)) != 0))
      return F8LIN_EINVAL;  // entries must share X, its copies, its state, the workspace and the events
    if (!aligned4(a.y_amax)) return F8LIN_EALIGN;
    const bool reuse = a.w_cast_valid != 0;
    if (reuse) {
      if (!a.sw.scale) return F8LIN_EINVAL;
    } else {
      F8_TRY(check_mode(a.mode_w));
      F8_TRY(check_state(a.sw, a.mode_w));
    }
    if (bad_dim(a.N) || a.N * K > kMaxElems || M * a.N > kMaxElems) return F8LIN_ESHAPE;
    const int64_t nk = a.N * K, mn = M * a.N, nkt = K * transposed_ld(a.N);
    if ((!reuse && missing(a.w, nk)) || missing(a.w8, nk) || missing(a.w8t, nk) || missing(a.y, mn))
      return F8LIN_EINVAL;
    if ((!reuse && !aligned16(a.w)) || !aligned16(a.y) || !aligned16(a.w8) || !aligned16(a.w8t) ||
        !aligned16(a.bias))
      return F8LIN_EALIGN;
    outs[no++] = {a.y, 2 * mn};
    outs[no++] = {a.y_amax, a.y_amax ? 4 : 0};
    if (reuse) {
      ins[ni++] = {a.w8, nk};
      ins[ni++] = {a.w8t, nkt};
      ins[ni++] = {a.sw.scale, 8};
    } else {
      need_ws = need_ws || a.mode_w == F8LIN_DYNAMIC;
      outs[no++] = {a.w8, nk};
      outs[no++] = {a.w8t, nkt};
      outs[no++] = {a.sw.scale, 8};
      outs[no++] = {a.sw.amax, 4};
      ins[ni++] = {a.w, 2 * nk};
      ins[ni++] = {a.sw.history, a.mode_w == F8LIN_DELAYED ? 64 : 0};
    }
    ins[ni++] = {a.bias, a.bias ? 2 * a.N : 0};
  }
  if (need_ws) {
    F8_TRY(check_ws(a0.ws, a0.ws_bytes));
    outs[no++] = {a0.ws, (int64_t)kWorkspaceBytes};
  }
  if (any_overlap(outs, no, ins, ni)) return F8LIN_EINVAL;

  hipStream_t s = (hipStream_t)stream;
  uint32_t *ws = (uint32_t *)a0.ws;
  // The output-amax words, zeroed by the first cast launch (X is always cast).
  ZeroWords zero;
  for (int i = 0; i < count; ++i)
    if (list[i].y_amax) zero.w[zero.n++] = list[i].y_amax;
  // The tensors to cast, dynamic-mode ones first (X leads its pass).
  CastTensor ct[1 + kMaxGemms];
  int modes[1 + kMaxGemms], nt = 0;
  bool given[1 + kMaxGemms] = {};
  for (int pass = 0; pass < 2; ++pass) {
    const int mode = pass == 0 ? F8LIN_DYNAMIC : F8LIN_DELAYED;
    if (a0.mode_x == mode) {
      given[nt] = x_given;
      ct[nt] = CastTensor{a0.x, M, K, &a0.sx, a0.x8, a0.x8t};
      ct[nt].ldt = transposed_ld(M);
      modes[nt++] = mode;
    }
    for (int i = 0; i < count; ++i) {
      const f8lin_fwd_args &a = list[i];
      if (!a.w_cast_valid && a.mode_w == mode) {
        ct[nt] = CastTensor{a.w, a.N, K, &a.sw, a.w8, a.w8t};
        ct[nt].ldt = transposed_ld(a.N);
        modes[nt++] = mode;
      }
    }
  }
  for (int i = 0; i < nt;) {
    const int n = (i + 1 < nt && modes[i + 1] == modes[i]) ? 2 : 1;
    CastTensor pair[2] = {ct[i], n > 1 ? ct[i + 1] : ct[i]};
    if (modes[i] == F8LIN_DYNAMIC) {
      // amax passes for the tensors whose amax is not handed in; when all of
      // them are small, the cast computes them itself (no amax launch)
      AmaxTensor am[2];
      int slot[2], na = 0;
      bool all_small = true;
      for (int j = 0; j < n; ++j)
        if (!given[i + j]) {
          slot[na] = j;
          am[na++] = AmaxTensor{pair[j].x, pair[j].rows * pair[j].cols, pair[j].st->amax};
          all_small = all_small && pair[j].rows * pair[j].cols <= kSelfAmaxElems;
        }
      if (na > 0 && all_small) {
        for (int j = 0; j < na; ++j) pair[slot[j]].self_amax = 1;
        na = 0;
      }
      if (na > 0 && a0.algo == F8LIN_AMAX_TWOPASS) {
        const uint32_t *parts[2] = {nullptr, nullptr};
        int nparts[2] = {0, 0};
        F8_TRY(status_of(launch_amax_partials(am, na, ws, parts, nparts, s)));
        for (int j = 0; j < na; ++j) pair[slot[j]].partials = parts[j], pair[slot[j]].npartials = nparts[j];
      } else if (na > 0) {
        F8_TRY(status_of(launch_amax(am, na, a0.algo, ws, s)));
      }
    }
    F8_TRY(status_of(launch_cast(pair, n, F8LIN_E4M3, modes[i], s, i == 0 ? zero : ZeroWords())));
    i += n;
  }
  GemmDesc g[kMaxGemms];
  for (int i = 0; i < count; ++i) {
    const f8lin_fwd_args &a = list[i];
    g[i] = GemmDesc{a0.x8, a.w8, a0.sx.scale + 1, a.sw.scale + 1, a.y, M, a.N, K, a.bias, a.y_amax};
  }
  F8_TRY(record(a0.ev_gemm_begin, s));
  F8_TRY(status_of(launch_gemms(g, count, F8LIN_E4M3, F8LIN_E4M3, s)));
  return record(a0.ev_gemm_end, s);
}

// Row tiles of the cast kernel: the number of per-tile column sums the bias
// gradient reduces (one when dY has no rows: that tile's sums are zeros).
int64_t dbias_tiles(int64_t M) { return M > 0 ? (M + kCastTile - 1) / kCastTile : 1; }

// ---- Scratch of f8lin_backward_noalloc, for callers that cannot allocate
// (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).  A file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current, and is kept per device.
//   [0, kWorkspaceBytes)       the workspace words (atomic-amax slots and
//                              tickets, two-pass partials, work-queue counters)
//   [kWorkspaceBytes, +16 MiB) the bias gradient's column sums, then the
//                              split GEMMs' fp32 partials (one after the other
//                              in stream order)
constexpr int kMaxDevices = 64;

__global__ void zero_words_kernel(uint32_t *p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x)) p[i] = 0u;
}

std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on the current device.  The first call on a
// device looks it up and clears the workspace words on `s` with a kernel
// (the array starts zeroed when the code object loads; every call leaves
// those words at zero again).
int static_scratch(uint8_t **out, hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return F8LIN_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(::scratch)) != hipSuccess || p == nullptr) return F8LIN_EHIP;
    zero_words_kernel<<<4, 256, 0, s>>>(reinterpret_cast<uint32_t *>(p), (int)(kWorkspaceBytes / 4));
    if (hipGetLastError() != hipSuccess) return F8LIN_EHIP;
    g_scratch_ptr[dev] = reinterpret_cast<uint8_t *>(p);
  }
  *out = g_scratch_ptr[dev];
  return F8LIN_OK;
}

// The backward.  lib_scratch: the caller passes no workspace, no bias-
// gradient scratch and no split scratch (all three must be NULL); the
// library's static scratch on the current device takes their place (the
// workspace words, and one region that the bias gradient's column sums and
// the split GEMMs' partials share: the sums are consumed by the dbias kernel
// before the GEMM launch writes any partial).
int backward_impl(const f8lin_bwd_args &in, void *stream, bool lib_scratch) {
  f8lin_bwd_args a = in;
  if (lib_scratch) {
    if (a.ws || a.dbias_ws || a.gemm_ws) return F8LIN_EINVAL;
    if (bad_dim(a.M) || bad_dim(a.N) || bad_dim(a.K)) return F8LIN_ESHAPE;
    if (a.dbias && f8lin_dbias_workspace_bytes(a.M, a.N) > kStaticRegionBytes) return F8LIN_EWORKSPACE;
  }
  if (!a.sx.scale || !a.sw.scale) return F8LIN_EINVAL;
  F8_TRY(check_mode(a.mode_dy));
  F8_TRY(check_algo(a.algo));
  F8_TRY(check_state(a.sdy, a.mode_dy));
  if (bad_dim(a.M) || bad_dim(a.N) || bad_dim(a.K) || a.M * a.K > kMaxElems || a.N * a.K > kMaxElems ||
      a.M * a.N > kMaxElems)
    return F8LIN_ESHAPE;
  if (missing(a.dy, a.M * a.N) || missing(a.dy8, a.M * a.N) || missing(a.dy8t, a.M * a.N) ||
      missing(a.x8t, a.M * a.K) || missing(a.dx, a.M * a.K) || missing(a.w8t, a.N * a.K) ||
      missing(a.dw, a.N * a.K))
    return F8LIN_EINVAL;
  if (!aligned16(a.dy) || !aligned16(a.x8t) || !aligned16(a.w8t) || !aligned16(a.dx) || !aligned16(a.dw) ||
      !aligned16(a.dy8) || !aligned16(a.dy8t) || !aligned16(a.dbias) || !aligned16(a.dbias_ws) ||
      !aligned16(a.gemm_ws))
    return F8LIN_EALIGN;
  // the part of gemm_ws that split GEMMs may write
  const int64_t gemm_ws = a.gemm_ws ? (int64_t)std::min<size_t>(a.gemm_ws_bytes,
                                                                 f8lin_backward_gemm_workspace_bytes(a.M, a.N, a.K))
                                    : 0;
  // dynamic mode needs the workspace for the amax; in either mode a valid one
  // also carries the GEMM's work queue (delayed mode may pass none)
  const bool dy_given = a.dy_amax_given != 0;
  if (dy_given && a.mode_dy != F8LIN_DYNAMIC) return F8LIN_EINVAL;
  if (!aligned4(a.dx_amax)) return F8LIN_EALIGN;
  const bool need_ws = a.mode_dy == F8LIN_DYNAMIC && !dy_given;
  if (need_ws && !lib_scratch) F8_TRY(check_ws(a.ws, a.ws_bytes));
  const bool use_ws = lib_scratch || need_ws || check_ws(a.ws, a.ws_bytes) == F8LIN_OK;
  const int64_t db_ws = a.dbias ? (int64_t)f8lin_dbias_workspace_bytes(a.M, a.N) : 0;
  if (!lib_scratch && db_ws > 0 && (!a.dbias_ws || a.dbias_ws_bytes < (size_t)db_ws)) return F8LIN_EWORKSPACE;
  const int64_t mk = a.M * a.K, nk = a.N * a.K, mn = a.M * a.N;
  const int64_t ld_m = transposed_ld(a.M), ld_n = transposed_ld(a.N);  // row strides of the transposed copies
  const Range outs[11] = {{a.dx, 2 * mk},
                          {a.dw, 2 * nk},
                          {a.dy8, mn},
                          {a.dy8t, a.N * ld_m},
                          {a.sdy.scale, 8},
                          {a.sdy.amax, dy_given ? 0 : 4},
                          {a.ws, use_ws && !lib_scratch ? (int64_t)kWorkspaceBytes : 0},
                          {a.dbias, a.dbias ? 2 * a.N : 0},
                          {a.dbias_ws, lib_scratch ? 0 : db_ws},
                          {a.gemm_ws, gemm_ws},
                          {a.dx_amax, a.dx_amax ? 4 : 0}};
  const Range ins[7] = {{a.dy, 2 * mn},  {a.x8t, a.K * ld_m}, {a.w8t, a.K * ld_n},
                        {a.sx.scale, 8}, {a.sw.scale, 8}, {a.sdy.history, a.mode_dy == F8LIN_DELAYED ? 64 : 0},
                        {a.sdy.amax, dy_given ? 4 : 0}};
  if (any_overlap(outs, 11, ins, 7)) return F8LIN_EINVAL;

  hipStream_t s = (hipStream_t)stream;
  int64_t gemm_ws_use = gemm_ws;
  if (lib_scratch) {  // every argument is valid: set up (first call on this device) and use the scratch
    uint8_t *sp = nullptr;
    F8_TRY(static_scratch(&sp, s));
    a.ws = sp;
    a.ws_bytes = kWorkspaceBytes;
    uint8_t *region = sp + kWorkspaceBytes;
    a.dbias_ws = a.dbias ? reinterpret_cast<float *>(region) : nullptr;
    a.dbias_ws_bytes = a.dbias ? kStaticRegionBytes : 0;
    a.gemm_ws = region;
    a.gemm_ws_bytes = kStaticRegionBytes;
    gemm_ws_use = (int64_t)std::min<size_t>(kStaticRegionBytes, f8lin_backward_gemm_workspace_bytes(a.M, a.N, a.K));
  }
  uint32_t *ws = (uint32_t *)a.ws;
  CastTensor cdy = {a.dy, a.M, a.N, &a.sdy, a.dy8, a.dy8t};
  cdy.ldt = ld_m;
  if (a.dbias) cdy.colsum = a.dbias_ws;  // the cast also sums dY's columns per 128-row tile
  if (a.mode_dy == F8LIN_DYNAMIC && !dy_given && mn <= kSelfAmaxElems) {
    cdy.self_amax = 1;  // small dY: the cast computes its amax itself
  } else if (a.mode_dy == F8LIN_DYNAMIC && !dy_given) {
    const AmaxTensor t = {a.dy, mn, a.sdy.amax};
    if (a.algo == F8LIN_AMAX_TWOPASS)
      F8_TRY(status_of(launch_amax_partials(&t, 1, ws, &cdy.partials, &cdy.npartials, s)));
    else
      F8_TRY(status_of(launch_amax(&t, 1, a.algo, ws, s)));
  }
  ZeroWords zero;
  if (a.dx_amax) zero.w[zero.n++] = a.dx_amax;
  F8_TRY(status_of(launch_cast(&cdy, 1, F8LIN_E5M2, a.mode_dy, s, zero)));
  if (a.dbias) F8_TRY(status_of(launch_dbias(a.dbias_ws, dbias_tiles(a.M), a.N, a.dbias, s)));
  // One launch for both GEMMs:
  //   dX (M, K) = dY8 (M, N) . [W8^T (K, N)]^T : contraction over N;
  //   dW (N, K) = dY8^T (N, M) . [X8^T (K, M)]^T : contraction over M.
  GemmDesc g[2] = {{a.dy8, a.w8t, a.sdy.scale + 1, a.sw.scale + 1, a.dx, a.M, a.K, a.N},
                   {a.dy8t, a.x8t, a.sdy.scale + 1, a.sx.scale + 1, a.dw, a.N, a.K, a.M}};
  g[0].amax_out = a.dx_amax;
  g[0].ldb = ld_n;  // W8^T (K, N)
  g[1].lda = ld_m;  // dY8^T (N, M)
  g[1].ldb = ld_m;  // X8^T (K, M)
  F8_TRY(record(a.ev_gemm_begin, s));
  F8_TRY(status_of(launch_gemms(g, 2, F8LIN_E5M2, F8LIN_E4M3, s, a.gemm_ws, (size_t)gemm_ws_use,
                                use_ws ? ws + kWsQueueOffset : nullptr)));
  return record(a.ev_gemm_end, s);
}


}  // namespace
}  // namespace f8lin

using namespace f8lin;

extern "C" {

size_t f8lin_workspace_bytes(void) { return kWorkspaceBytes; }

int64_t f8lin_transposed_ld(int64_t rows) { return rows < 0 ? 0 : transposed_ld(rows); }

size_t f8lin_dbias_workspace_bytes(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return 0;
  return (size_t)dbias_tiles(M) * (size_t)N * sizeof(float);
}

size_t f8lin_backward_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return 0;
  // dgrad: (M, K) contracted over N; wgrad: (N, K) contracted over M
  return split_workspace_bytes(M, K, N) + split_workspace_bytes(N, K, M);
}

const char *f8lin_status_str(int status) {
  switch (status) {
    case F8LIN_OK: return "F8LIN_OK";
    case F8LIN_EINVAL: return "F8LIN_EINVAL: invalid argument (null pointer, enum, overlap or count)";
    case F8LIN_ESHAPE: return "F8LIN_ESHAPE: dimension negative, too large, or not a multiple of 16";
    case F8LIN_EALIGN: return "F8LIN_EALIGN: pointer not 16-byte aligned";
    case F8LIN_EWORKSPACE: return "F8LIN_EWORKSPACE: workspace missing, misaligned or too small";
    case F8LIN_EHIP: return "F8LIN_EHIP: HIP launch failed";
    default: return "unknown f8lin status";
  }
}

int f8lin_amax(const uint16_t *x, int64_t n, int algo, float *amax_out, void *ws, size_t ws_bytes,
               void *stream) {
  if (!amax_out) return F8LIN_EINVAL;
  F8_TRY(check_algo(algo));
  if (n < 0 || n > kMaxElems) return F8LIN_ESHAPE;
  if (missing(x, n)) return F8LIN_EINVAL;
  if (!aligned16(x)) return F8LIN_EALIGN;
  F8_TRY(check_ws(ws, ws_bytes));
  const Range outs[2] = {{amax_out, 4}, {ws, (int64_t)kWorkspaceBytes}};
  const Range ins[1] = {{x, 2 * n}};
  if (any_overlap(outs, 2, ins, 1)) return F8LIN_EINVAL;
  const AmaxTensor t = {x, n, amax_out};
  return status_of(launch_amax(&t, 1, algo, (uint32_t *)ws, (hipStream_t)stream));
}

int f8lin_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, int fmt, int mode,
                         const f8lin_state *st, uint8_t *q, uint8_t *qt, void *stream) {
  F8_TRY(validate_cast(x, rows, cols, fmt, mode, st, q, qt));
  CastTensor t = {x, rows, cols, st, q, qt};
  t.ldt = transposed_ld(rows);
  return status_of(launch_cast(&t, 1, fmt, mode, (hipStream_t)stream));
}

int f8lin_cast_f32(const float *v, int64_t n, int fmt, uint8_t *q, void *stream) {
  F8_TRY(check_fmt(fmt));
  if (n < 0 || n > kMaxElems) return F8LIN_ESHAPE;
  if (missing(v, n) || missing(q, n)) return F8LIN_EINVAL;
  if (!aligned16(v) || !aligned16(q)) return F8LIN_EALIGN;
  const Range outs[1] = {{q, n}};
  const Range ins[1] = {{v, 4 * n}};
  if (any_overlap(outs, 1, ins, 1)) return F8LIN_EINVAL;
  return status_of(launch_cast_f32(v, n, fmt, q, (hipStream_t)stream));
}

int f8lin_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N, int64_t K,
               const float *inv_scale_a, const float *inv_scale_b, uint16_t *c, void *stream) {
  F8_TRY(validate_gemm(a, fmt_a, b, fmt_b, M, N, K, inv_scale_a, inv_scale_b, c));
  return status_of(launch_gemm(a, fmt_a, b, fmt_b, M, N, K, inv_scale_a, inv_scale_b, c, (hipStream_t)stream));
}

int f8lin_gemm_batch(const f8lin_gemm_desc *d, int count, int fmt_a, int fmt_b, void *stream) {
  static_assert(F8LIN_MAX_BATCH == kMaxGemms, "batch limit");
  if (!d || count < 1 || count > F8LIN_MAX_BATCH) return F8LIN_EINVAL;
  GemmDesc g[kMaxGemms];
  Range outs[kMaxGemms], ins[4 * kMaxGemms];
  for (int i = 0; i < count; ++i) {
    const f8lin_gemm_desc &e = d[i];
    F8_TRY(validate_gemm(e.a, fmt_a, e.b, fmt_b, e.M, e.N, e.K, e.inv_scale_a, e.inv_scale_b, e.c, e.lda, e.ldb));
    g[i] = GemmDesc{e.a, e.b, e.inv_scale_a, e.inv_scale_b, e.c, e.M, e.N, e.K};
    g[i].lda = e.lda ? e.lda : e.K;
    g[i].ldb = e.ldb ? e.ldb : e.K;
    outs[i] = Range{e.c, 2 * e.M * e.N};
    ins[4 * i] = Range{e.a, e.M * g[i].lda};
    ins[4 * i + 1] = Range{e.b, e.N * g[i].ldb};
    ins[4 * i + 2] = Range{e.inv_scale_a, 4};
    ins[4 * i + 3] = Range{e.inv_scale_b, 4};
  }
  if (any_overlap(outs, count, ins, 4 * count)) return F8LIN_EINVAL;
  return status_of(launch_gemms(g, count, fmt_a, fmt_b, (hipStream_t)stream));
}

int f8lin_forward(const f8lin_fwd_args *p, void *stream) { return forward_impl(p, 1, stream); }

int f8lin_forward_shared_x(const f8lin_fwd_args *args, int count, void *stream) {
  return forward_impl(args, count, stream);
}

int f8lin_backward(const f8lin_bwd_args *p, void *stream) {
  if (!p) return F8LIN_EINVAL;
  return backward_impl(*p, stream, false);
}

int f8lin_backward_noalloc(const f8lin_bwd_args *p, void *stream) {
  if (!p) return F8LIN_EINVAL;
  return backward_impl(*p, stream, true);
}

int f8lin_delayed_update(const f8lin_state *states, int n_states, int32_t *status, void *stream) {
  if (!states || n_states < 0) return F8LIN_EINVAL;
  if (!aligned4(status)) return F8LIN_EALIGN;
  for (int i = 0; i < n_states; ++i) {
    const f8lin_state &st = states[i];
    if (!st.amax || !st.history || !st.hist_meta) return F8LIN_EINVAL;
    if (!aligned16(st.history) || !aligned4(st.amax) || !aligned4(st.hist_meta)) return F8LIN_EALIGN;
    // the status words are written: they must not overlap any state
    const Range out = {status, status ? 4 * (int64_t)n_states : 0};
    const Range st_r[3] = {{st.amax, 4}, {st.history, 64}, {st.hist_meta, 8}};
    if (any_overlap(&out, 1, st_r, 3)) return F8LIN_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  for (int i0 = 0; i0 < n_states; i0 += kUpdateBatch) {
    StateBatch b;
    memset(&b, 0, sizeof b);
    b.n = n_states - i0 < kUpdateBatch ? n_states - i0 : kUpdateBatch;
    for (int i = 0; i < b.n; ++i) b.s[i] = states[i0 + i];
    delayed_update_kernel<<<1, 64, 0, s>>>(b, status ? status + i0 : nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return F8LIN_EHIP;
  }
  return F8LIN_OK;
}

}  // extern "C"
