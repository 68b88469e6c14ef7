// Scale + saturating fp8 cast of a bf16 (rows, cols) tensor, writing the
// row-major codes q and the transposed codes qt in one pass (the backward
// GEMMs contract over the other dimension and read qt).
//
// Tensorwise scaling (pytorch/torchtitan PR #778 Summary: tensorwise dynamic
// scaling; pytorch/ao issue #1297 repro: delayed scaling of input, weight and
// grad_output).  The scale is computed in every workgroup's prologue from the
// state (dynamic: state.amax, or the per-workgroup partial maxima of the
// two-pass amax, which each workgroup reduces itself -- the second pass of
// that algorithm -- so it needs no launch of its own; delayed: max of the
// 16-entry amax history), so no extra launch and no host round trip sit
// between amax and cast.
//
// Work decomposition (gfx950, wave64): one workgroup of 256 threads per
// 128 x 128 tile; one launch may cast two tensors (the forward's X and W).
//   load   : thread t reads 16 consecutive bf16 (two 128-bit loads) of rows
//            t/8 + 32p, p = 0..3; eight threads cover one 256-byte row segment.
//   q      : the 16 codes go out as one 128-bit store (a 128-byte row segment
//            per 8 threads) and into LDS.
//   qt     : thread (k = t%8, g = t/8) reads the 4-byte column group g of the
//            16 tile rows 16k..16k+15 from LDS, transposes the four 4x4 byte
//            blocks in registers (v_perm_b32), and writes four 128-bit qt
//            stores; eight neighbouring threads fill one 128-byte qt segment.
//            qt's rows are ldt bytes apart (rows, or rows + 128 when rows is
//            a multiple of 32768: see transposed_ld).
//   LDS    : 128 rows x 128 bytes, 16-byte chunks XOR-swizzled by
//            (row / 16) % 8, which makes both the 128-bit row writes and the
//            4-byte column reads spread over all banks.
// Delayed mode also folds max |x| into state.amax (atomic max on the fp32
// bit pattern, which orders like the value for non-negative floats).  Same-
// address atomics serialise (one per tile cost 6-16 us per cast at 1248-5450
// tiles, measured), so a delayed-mode workgroup takes two tiles -- two
// independent 256-thread halves, each as above -- and issues one atomic (two
// tiles beat four by 12-16% at 1248-4800 tiles, where four leave a coarse
// last wave of workgroups; the same elsewhere).
//
// HBM-bound: 2 bytes read + 2 bytes written per element (4 B/elem).
#include "device_common.h"
#include "internal.h"

namespace f8lin {
namespace {

constexpr int kTile = kCastTile;
constexpr int kThreads = 256;
static_assert(kThreads / 64 == 4 && kMaxGrid <= kThreads, "partials reduction layout");

__device__ __forceinline__ int lds_word(int row, int word) {
  // 32 words per row; 16-byte chunk index XOR (row / 16) % 8.
  return row * 32 + ((((word >> 2) ^ (row >> 4)) & 7) << 2) + (word & 3);
}

// Transposes a 4x4 byte block: d[r] holds bytes (r, 0..3); returns e[c]
// holding bytes (0..3, c).
__device__ __forceinline__ void transpose4x4(const uint32_t d0, const uint32_t d1, const uint32_t d2,
                                             const uint32_t d3, uint32_t &e0, uint32_t &e1, uint32_t &e2,
                                             uint32_t &e3) {
  // v_perm_b32(hi, lo, sel): selector byte 0-3 picks lo's bytes, 4-7 hi's.
  const uint32_t t0 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);  // d0.0 d1.0 d0.1 d1.1
  const uint32_t t1 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);  // d0.2 d1.2 d0.3 d1.3
  const uint32_t t2 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);  // d2.0 d3.0 d2.1 d3.1
  const uint32_t t3 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);  // d2.2 d3.2 d2.3 d3.3
  e0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);                 // d0.0 d1.0 d2.0 d3.0
  e1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);                 // d0.1 d1.1 d2.1 d3.1
  e2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);                 // d0.2 d1.2 d2.2 d3.2
  e3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);                 // d0.3 d1.3 d2.3 d3.3
}

// Up to two tensors per launch (the forward casts X and W together):
// workgroups [first[i], first[i] + tiles[i]) take tensor i's tiles.
struct CastJob {
  const uint16_t *x;
  int64_t rows, cols;
  float *amax;            // dynamic: this tensor's amax (written here when partials are given)
  const uint32_t *partials;  // dynamic, two-pass: the partial magnitude maxima, or null
  int npartials;
  int self_amax;          // dynamic, small tensor: every workgroup reduces the whole tensor itself
  const float *history;   // delayed: its amax history
  float *amax_acc;        // delayed: where this step's amax accumulates
  float *scale_out;       // {scale, 1/scale}
  uint8_t *q, *qt;
  int64_t ldt;            // row stride of qt (bytes)
  float *colsum;          // per-tile column sums (bias gradient), or null
  int tiles_x;
  int first;              // first workgroup of this tensor
  int ntiles;
};
struct CastJobs {
  CastJob j[2];
  int count;
  ZeroWords zero;  // set to +0 by the first workgroup
};

// TPW tiles per workgroup: the 256 threads of part `sub` cast tile
// first_tile + sub; a part past the tensor's last tile loads and stores
// nothing.
template <int FMT, int MODE, bool WRITE_T, int TPW>
__global__ __launch_bounds__(kThreads * TPW) void cast_transpose_kernel(const CastJobs jobs) {
  __shared__ uint32_t tiles_lds[TPW][kTile * kTile / 4];
  __shared__ uint32_t red[kThreads * TPW / 64];
  __shared__ float colred[TPW][kThreads / 64][kTile];
  constexpr float fm = fmt_max<FMT>();
  const int job = (jobs.count > 1 && (int)blockIdx.x >= jobs.j[1].first) ? 1 : 0;
  const CastJob &jb = jobs.j[job];
  const uint16_t *__restrict__ x = jb.x;
  const int64_t rows = jb.rows, cols = jb.cols;
  uint8_t *__restrict__ q = jb.q;
  uint8_t *__restrict__ qt = jb.qt;
  const int sub = TPW > 1 ? (int)(threadIdx.x / kThreads) : 0;
  const int local = ((int)blockIdx.x - jb.first) * TPW + sub;  // this part's tile
  const int t = threadIdx.x % kThreads;
  const int c16 = t & 7;
  const int rsub = t >> 3;
  const bool want_cs = jb.colsum != nullptr;

  // The scale's inputs are read before the tile, so that waiting for them
  // does not also wait for the tile's loads (measured: -1 us per cast at
  // 4096 x 4096).
  uint32_t pmag = 0;
  float a = 0.0f;
  if constexpr (MODE == F8LIN_DYNAMIC) {
    if (jb.partials) {
      pmag = t < jb.npartials ? jb.partials[t] : 0u;  // at most kMaxGrid <= kThreads partials
    } else if (!jb.self_amax) {
      a = jb.amax[0];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kHistLen; ++i) {
      const float h = jb.history[i];
      a = (h != h || a != a) ? __builtin_nanf("") : fmaxf(a, h);
    }
  }

  // Loads the tile; then, once the scale is known, converts and stores it
  // (the tile's addresses are recomputed there rather than kept live across
  // the scale's barriers: fewer registers, which keeps four waves per SIMD).
  auto load = [&](u32x4(&in)[4][2]) {
    const int64_t row0 = (int64_t)(local / jb.tiles_x) * kTile;
    const int64_t gcol = (int64_t)(local % jb.tiles_x) * kTile + c16 * 16;
    const bool col_ok = local < jb.ntiles && gcol < cols;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t grow = row0 + rsub + 32 * p;
      if (col_ok && grow < rows) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + grow * cols + gcol);
        in[p][0] = src[0];
        in[p][1] = src[1];
      } else {
        in[p][0] = u32x4{0, 0, 0, 0};
        in[p][1] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto cast_tile = [&](const u32x4(&in)[4][2], float s) {
    uint32_t *tile = tiles_lds[sub];
    const bool live = local < jb.ntiles;
    const int64_t row0 = (int64_t)(local / jb.tiles_x) * kTile;
    const int64_t col0 = (int64_t)(local % jb.tiles_x) * kTile;
    const int64_t gcol = col0 + c16 * 16;
    const bool col_ok = live && gcol < cols;

    // Column sums of this thread's four rows (bias gradient), in row order.
    float cs[16];
    if (want_cs) {
#pragma unroll
      for (int e = 0; e < 16; ++e) cs[e] = 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w4[4] = {in[p][h].x, in[p][h].y, in[p][h].z, in[p][h].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            cs[8 * h + 2 * w] += bf16_lo(w4[w]);
            cs[8 * h + 2 * w + 1] += bf16_hi(w4[w]);
          }
        }
    }

    uint32_t mag = 0;
  #pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = rsub + 32 * p;
      const int64_t grow = row0 + r;
      u32x4 o;
      o.x = quantize4<FMT>(in[p][0].x, in[p][0].y, s);
      o.y = quantize4<FMT>(in[p][0].z, in[p][0].w, s);
      o.z = quantize4<FMT>(in[p][1].x, in[p][1].y, s);
      o.w = quantize4<FMT>(in[p][1].z, in[p][1].w, s);
      if constexpr (MODE == F8LIN_DELAYED) {
        mag = mag_max2(mag, in[p][0].x);
        mag = mag_max2(mag, in[p][0].y);
        mag = mag_max2(mag, in[p][0].z);
        mag = mag_max2(mag, in[p][0].w);
        mag = mag_max2(mag, in[p][1].x);
        mag = mag_max2(mag, in[p][1].y);
        mag = mag_max2(mag, in[p][1].z);
        mag = mag_max2(mag, in[p][1].w);
      }
      if (col_ok && grow < rows) *reinterpret_cast<u32x4 *>(q + grow * cols + gcol) = o;
      if constexpr (WRITE_T) *reinterpret_cast<u32x4 *>(&tile[lds_word(r, c16 * 4)]) = o;
    }

    if constexpr (MODE == F8LIN_DELAYED) {
      // Out-of-range elements were loaded as +0 and cannot raise the max.
  #pragma unroll
      for (int off = 32; off > 0; off >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off, 64));
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mag;
    }

    if constexpr (WRITE_T || MODE == F8LIN_DELAYED) __syncthreads();

    if constexpr (MODE == F8LIN_DELAYED) {
      if (threadIdx.x == 0) {  // one atomic for the workgroup's TPW tiles
        uint32_t m = red[0];
  #pragma unroll
        for (int w = 1; w < kThreads * TPW / 64; ++w) m = max(m, red[w]);
        atomicMax(reinterpret_cast<uint32_t *>(jb.amax_acc), m << 16);
      }
    }

    if constexpr (WRITE_T) {
      const int k = t & 7;   // 16-row group of the tile
      const int g = t >> 3;  // 4-column group of the tile
      const int64_t qrow = col0 + 4 * g;  // first of the four qt rows
      const int64_t qcol = row0 + 16 * k;
      uint32_t d[16];
  #pragma unroll
      for (int i = 0; i < 16; ++i) d[i] = tile[lds_word(16 * k + i, g)];
      u32x4 out[4];
  #pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t e0, e1, e2, e3;
        transpose4x4(d[4 * m], d[4 * m + 1], d[4 * m + 2], d[4 * m + 3], e0, e1, e2, e3);
        out[0][m] = e0;
        out[1][m] = e1;
        out[2][m] = e2;
        out[3][m] = e3;
      }
      if (live && qrow < cols && qcol < rows) {
  #pragma unroll
        for (int b = 0; b < 4; ++b) *reinterpret_cast<u32x4 *>(qt + (qrow + b) * jb.ldt + qcol) = out[b];
      }
    }
    // Bias gradient: this tile's column sums.  The 32 threads of one column
    // group are lanes c16 + 8 * (0..7) of the four waves: a fixed xor tree
    // inside each wave, then the four waves in order -- the same order on
    // every run.
    if (want_cs) {
  #pragma unroll
      for (int off = 8; off < 64; off <<= 1)
  #pragma unroll
        for (int e = 0; e < 16; ++e) cs[e] += __shfl_xor(cs[e], off, 64);
      const int lane = t & 63, wave = t >> 6;
      if (lane < 8) {
  #pragma unroll
        for (int e = 0; e < 16; ++e) colred[sub][wave][lane * 16 + e] = cs[e];
      }
      __syncthreads();
      if (live && t < kTile && col0 + t < cols) {
        const float v = ((colred[sub][0][t] + colred[sub][1][t]) + colred[sub][2][t]) + colred[sub][3][t];
        jb.colsum[(row0 / kTile) * cols + col0 + t] = v;
      }
    }
  };

  u32x4 in[4][2];
  load(in);
  if constexpr (MODE == F8LIN_DYNAMIC) {
    if (jb.self_amax) {
      // A small tensor (at most kSelfAmaxElems elements, whole 8-element
      // vectors since cols is a multiple of 16): every workgroup reads all of
      // it -- from the L2 once the first has -- instead of a separate amax
      // launch; the same 15-bit magnitude max, so the same bits.
      const u32x4 *__restrict__ xv = reinterpret_cast<const u32x4 *>(x);
      const int nv = (int)(rows * cols / 8);
      int i = t;
      for (; i + 7 * kThreads < nv; i += 8 * kThreads) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = xv[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pmag = mag_max2(mag_max2(mag_max2(mag_max2(pmag, v[u].x), v[u].y), v[u].z), v[u].w);
      }
      for (; i < nv; i += kThreads) {
        const u32x4 v = xv[i];
        pmag = mag_max2(mag_max2(mag_max2(mag_max2(pmag, v.x), v.y), v.z), v.w);
      }
    }
  }

  // The scale.
  if constexpr (MODE == F8LIN_DYNAMIC) {
    if (jb.partials || jb.self_amax) {
      uint32_t m = pmag;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
      if ((t & 63) == 0) red[t >> 6] = m;
      __syncthreads();
      m = max(max(red[0], red[1]), max(red[2], red[3]));
      a = __uint_as_float(m << 16);
      __syncthreads();  // red is reused by the delayed-mode reduction below
      if (local == 0 && t == 0) jb.amax[0] = a;
    }
  }
  const float s = scale_from_amax(a, fm);
  if (local == 0 && t == 0) {
    jb.scale_out[0] = s;
    jb.scale_out[1] = 1.0f / s;
  }
  if (blockIdx.x == 0 && threadIdx.x < (unsigned)jobs.zero.n) jobs.zero.w[threadIdx.x][0] = 0.0f;
  cast_tile(in, s);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void cast_f32_kernel(const float *__restrict__ v, int64_t n,
                                                            uint8_t *__restrict__ q) {
  constexpr float fm = fmt_max<FMT>();
  const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 f = *reinterpret_cast<const float4 *>(v + i);
    *reinterpret_cast<uint32_t *>(q + i) =
        cvt4<FMT>(saturate(f.x, fm), saturate(f.y, fm), saturate(f.z, fm), saturate(f.w, fm));
  } else {
    for (int64_t j = i; j < n; ++j) q[j] = (uint8_t)(cvt4<FMT>(saturate(v[j], fm), 0.f, 0.f, 0.f) & 0xFFu);
  }
}

// Bias gradient from the per-tile column sums: workgroup of 256 threads per
// 32 columns; thread (column c, group g) sums tiles g, g + 8, ... in order,
// then thread (c, 0) adds the eight group sums in order: a fixed order on
// every run.
constexpr int kDbCols = 32, kDbGroups = 8;
__global__ __launch_bounds__(kDbCols * kDbGroups) void dbias_kernel(const float *__restrict__ colsum, int64_t tiles,
                                                                     int64_t n, uint16_t *__restrict__ db) {
  __shared__ float part[kDbGroups][kDbCols];
  const int c = threadIdx.x % kDbCols, g = threadIdx.x / kDbCols;
  const int64_t col = (int64_t)blockIdx.x * kDbCols + c;
  float s = 0.0f;
  if (col < n) {
    int64_t t = g;
    for (; t + 7 * kDbGroups < tiles; t += 8 * kDbGroups) {  // eight loads in flight, added in order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = colsum[(t + u * kDbGroups) * n + col];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; t < tiles; t += kDbGroups) s += colsum[t * n + col];
  }
  part[g][c] = s;
  __syncthreads();
  if (g == 0 && col < n) {
    float r = part[0][c];
#pragma unroll
    for (int i = 1; i < kDbGroups; ++i) r += part[i][c];
    db[col] = (uint16_t)f32_to_bf16_rne(r);
  }
}

// Tiles per workgroup: two in delayed mode (one atomic per two tiles), one
// in dynamic mode.
template <int MODE>
constexpr int tiles_per_wg() { return MODE == F8LIN_DELAYED ? 2 : 1; }

template <int FMT, int MODE>
void launch_ct(unsigned grid, const CastJobs &jobs, bool write_t, hipStream_t stream) {
  constexpr int TPW = tiles_per_wg<MODE>();
  if (write_t)
    cast_transpose_kernel<FMT, MODE, true, TPW><<<grid, kThreads * TPW, 0, stream>>>(jobs);
  else
    cast_transpose_kernel<FMT, MODE, false, TPW><<<grid, kThreads * TPW, 0, stream>>>(jobs);
}

}  // namespace

hipError_t launch_cast(const CastTensor *ts, int count, int fmt, int mode, hipStream_t stream,
                       const ZeroWords &zero) {
  // Every tensor gets at least one workgroup, even when empty: it still
  // publishes the scale.  (The C-ABI layer bounds rows * cols, so the tile
  // count fits a 1-D grid.)  The transposed copy is written for all tensors
  // of a launch or for none.
  CastJobs jobs = {};
  jobs.count = count;
  jobs.zero = zero;
  const int64_t tpw = mode == F8LIN_DELAYED ? tiles_per_wg<F8LIN_DELAYED>() : tiles_per_wg<F8LIN_DYNAMIC>();
  int64_t total = 0;  // workgroups
  for (int i = 0; i < count; ++i) {
    const CastTensor &t = ts[i];
    const int64_t gx = t.cols > 0 ? (t.cols + kTile - 1) / kTile : 1;
    const int64_t gy = t.rows > 0 ? (t.rows + kTile - 1) / kTile : 1;
    jobs.j[i] = CastJob{t.x,           t.rows,       t.cols,      t.st->amax,  t.partials,
                        t.npartials,   t.self_amax,  t.st->history, t.st->amax, t.st->scale,
                        t.q,           t.qt,         t.ldt ? t.ldt : t.rows,    t.colsum,
                        (int)gx,       (int)total,   (int)(gx * gy)};
    total += (gx * gy + tpw - 1) / tpw;
  }
  // (An empty tensor may pass a null qt; its workgroup writes no rows.)
  bool write_t = false;
  for (int i = 0; i < count; ++i) write_t = write_t || ts[i].qt != nullptr;
  const unsigned grid = (unsigned)total;
  if (fmt == F8LIN_E4M3) {
    if (mode == F8LIN_DYNAMIC) launch_ct<0, F8LIN_DYNAMIC>(grid, jobs, write_t, stream);
    else launch_ct<0, F8LIN_DELAYED>(grid, jobs, write_t, stream);
  } else {
    if (mode == F8LIN_DYNAMIC) launch_ct<1, F8LIN_DYNAMIC>(grid, jobs, write_t, stream);
    else launch_ct<1, F8LIN_DELAYED>(grid, jobs, write_t, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dbias(const float *colsum, int64_t tiles, int64_t n_cols, uint16_t *db, hipStream_t stream) {
  if (n_cols == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_cols + kDbCols - 1) / kDbCols);
  dbias_kernel<<<grid, kDbCols * kDbGroups, 0, stream>>>(colsum, tiles, n_cols, db);
  return hipGetLastError();
}

hipError_t launch_cast_f32(const float *v, int64_t n, int fmt, uint8_t *q, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 4 * kThreads - 1) / (4 * kThreads);
  if (fmt == F8LIN_E4M3)
    cast_f32_kernel<0><<<(unsigned)blocks, kThreads, 0, stream>>>(v, n, q);
  else
    cast_f32_kernel<1><<<(unsigned)blocks, kThreads, 0, stream>>>(v, n, q);
  return hipGetLastError();
}

}  // namespace f8lin
