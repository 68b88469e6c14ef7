// fp8 GEMM with a per-tensor dequantisation epilogue, for all three GEMMs of
// the Float8Linear forward + backward (pytorch/torchtitan PR #778,
// "Benchmarking single linear layer forward+backward performance"):
//   C (M, N) bf16 = (A (M, K) . B (N, K)^T) * inv_a * inv_b
// Both operands are K-contiguous ("TN"); the cast kernel writes the
// transposed fp8 copies so that forward, dgrad and wgrad all take this form.
// One launch runs a list of up to four such problems (the backward's dgrad
// and wgrad go together, so do the forwards of linears that share their
// input); problems with M <= 64 take a skinny kernel of their own (below).
//
// gfx950 design (each choice measured on MI355X):
//   * v_mfma_f32_16x16x128_f8f6f4 in the big tiles, v_mfma_f32_32x32x64_f8f6f4
//     in the others (the scaled builtins with zero scale operands select the
//     unscaled instructions); e4m3 / e5m2 per operand through cbsz / blgp.
//     A lane feeds the same 32 K-bytes of its A row and of its B row, so A
//     and B share one K order and the instruction's internal K order cannot
//     matter.  The matrix cores are power-bound on real data: on random fp8
//     codes from registers the 16 x 16 x 128 instruction runs ~10% more
//     flops per second than the 32 x 32 x 64 one (the chip holds ~2.04
//     instead of ~1.89 GHz): it moves half the accumulator data per flop.
//   * Workgroups:
//       big   256 x 256 tile, 4 waves (2 x 2, one per SIMD), wave tile
//             128 x 128 (256 fp32 accumulators per lane, in the AGPRs), one
//             workgroup per CU, with its own K loop (below); contractions
//             of fewer than four K blocks and split-K ranges of fewer than
//             16 take 8 waves instead (2 x 4, wave tile 128 x 64, two per
//             SIMD, the loop of the smaller tiles);
//       small 128 x 128 tile, 4 waves (2 x 2), wave tile 64 x 64, two per CU,
//             for problems with too few big tiles to fill 256 CUs, or
//             whose ragged edge would leave the last round of big tiles
//             nearly empty, and for the rows a lone problem has left over
//             after its full rounds of big tiles (a second launch);
//       medium 64 x 128 tile, 4 waves (2 x 2), wave tile 32 x 64, when even
//             the small tiles number fewer than the CUs (a few hundred
//             tokens): twice as many tiles, twice as many busy CUs.
//   * K block of 128 bytes in two LDS stages.  Global -> LDS copies use
//     buffer_load_dwordx4 ... lds (no register staging); eight lanes fetch
//     one full 128-byte row line (64-byte row segments, i.e. K blocks of 64,
//     loaded ~1.5x slower).  The buffer resource's range check returns zeros
//     for rows past M / N, and K chunks past K point outside the range, so
//     ragged edges load zeros with no branches.
//   * LDS slot of (row r, 16-byte chunk c) = r*8 + (c ^ ((r>>1) & 7)): every
//     16 consecutive rows at one chunk fall in 16 distinct bank groups, so
//     the 128-bit fragment reads are conflict-free.
//   * Schedule of the small and medium tiles (two waves per SIMD; fixed with
//     scheduling fences, since the compiler otherwise clusters the LDS reads
//     after the MFMAs and the waves stall on them): MFMAs go column by
//     column over the wave tile; each fragment register is refilled from LDS
//     right after its last MFMA, at least three MFMAs before its next use.
//     One barrier per K block sits after the first column of its second
//     half: it publishes block k+1 (each wave first waits for its own copies)
//     and retires block k, whose buffer then receives block k+2; those copies
//     are spread between the MFMAs that follow.
//   * The big tile's K loop (one wave per SIMD, so nothing hides a wave's
//     stall but its own schedule): each block's A fragments are read from
//     LDS during one 32-MFMA step and its B fragments during the next, so the
//     A and B regions of a stage are freed one step apart and each step
//     refills one region (eight 1 KB copies per wave): every step issues the
//     same share of copies, and a copy has two to three steps to land before
//     it is read.  A fragment is mostly read into the registers of the one it
//     replaces right after that one's last MFMA, so ~22 of them (176 VGPRs)
//     are live.  On 4096 x 4096 x 16384 this runs 6% faster than the same
//     loop on 32 x 32 x 64 MFMAs (same box).  Two waves per SIMD with a
//     128 x 64 wave tile read 1.5x the LDS bytes per flop and were slower
//     still.
//   * The matrix cores and the memory system together exceed the chip's power
//     budget: the shader clock drops from 2.4 GHz to ~1.7-2.0 GHz while this
//     loop runs (read with s_memtime against the constant-rate counter), so
//     bytes moved per flop cost time even when they are hidden.
//   * Persistent workgroups walk XCD-aware tile lists.  Workgroup b runs on
//     XCD b % 8 (round-robin dispatch), and each XCD has its own L2, so XCD x
//     owns a contiguous eighth of each problem's tile list, laid out in groups
//     of G tile-rows walked column by column: the tiles an XCD runs at once
//     form a compact patch whose A and B slices its L2 shares (4096^3: 96 MiB
//     read past L2 instead of 144 MiB with row-major order).  Giving every
//     XCD its share of every problem keeps a batch balanced when the problems'
//     K differ (wgrad's K is the token count).
//   * Output stores are non-temporal when a launch has four or more tiles per
//     CU, so that C does not push operand lines out of the caches.
//   * Epilogue: acc * (inv_a * inv_b) in fp32 (+ the bias in fp32, when the
//     layer has one: pytorch/ao issue #1297, repro script, whose nn.Linear
//     layers keep their default bias; its loads are range-checked buffer
//     loads issued together), then rounded to bf16 pairs by
//     v_cvt_pk_bf16_f32 (nearest even; checked against a software rounding on
//     all 2^32 binary32 patterns): the big tiles' MFMAs run on C^T, so a lane
//     already holds four adjacent columns, and in the other tiles a DPP swap
//     brings two adjacent columns into one lane.  The tile is staged through
//     LDS per wave and written as 16-byte row segments.
#include <algorithm>
#include <vector>

#include "device_common.h"
#include "internal.h"

namespace f8lin {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;
constexpr int kMinBigK = 4 * kBK;  // shortest K the 256 x 256 tiles take
#ifndef F8LIN_SPLIT_STAG_BLOCKS
#define F8LIN_SPLIT_STAG_BLOCKS 16
#endif
constexpr int kSplitStagBlocks = F8LIN_SPLIT_STAG_BLOCKS;  // shortest split range the four-wave tiles take
constexpr int kXcds = 8;
constexpr int kCUs = 256;
// Every matrix dimension is at most 2^22 (checked at the C ABI), so a tile's
// byte range rows * K stays below 2^31 and this offset is always outside it.
constexpr int kOutOfRange = (int)0x80000000u;

struct Problem {
  const uint8_t *a, *b;
  const float *inv_a, *inv_b;
  uint16_t *c;           // (M, N) bf16; split problems: splits x (M, N) fp32 partial sums
  const uint16_t *bias;  // (N) bf16 or null
  int M, N, K;
  int lda, ldb;  // row strides (bytes) of A and B, >= K
  int tiles_m, tiles_n;
  int splits;  // split problems: K-block ranges, each a partial product of its own
  float *amax_out;  // AMAX: max |C| (of the rounded bf16 values) folded in here, or null
};
struct Batch {
  Problem p[kMaxGemms];
  int count;
  int nt_stores;     // write C with non-temporal stores (many tiles per CU)
  uint32_t *queue;   // DYN: per-XCD work-queue words (zero at launch, left zero)
};

__device__ __forceinline__ int slot128(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// (tile-row, tile-column) of a problem's local tile index: groups of G
// tile-rows, each walked column by column.
template <int G>
__device__ __forceinline__ void tile_coords(int local, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int gsize = G * tiles_n;
  const int grp = local / gsize, in = local % gsize;
  const int gm = min(G, tiles_m - grp * G);
  tm = grp * G + in % gm;
  tn = in / gm;
}

template <bool B>
using bool_t = std::integral_constant<bool, B>;
template <int V>
using int_t = std::integral_constant<int, V>;
// The lane index (0-63), produced by an instruction the compiler cannot move:
// kernels at the register limit call this where they need it instead of
// keeping it live (a spilled value's reload waits for all memory operations
// in flight, copies and stores included).
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
// block parity of the step k steps after one of parity (p0, h0)
constexpr int step_p(int p0, int h0, int k) { return (p0 + ((h0 + k) >> 1)) & 1; }

// PARTIAL: every problem is split along K into P.splits ranges of whole K
// blocks; the tile list holds every (range, tile) pair, and a tile writes its
// range's fp32 partial product, unscaled, to slab `range` of P.c (summed,
// scaled and rounded by split_reduce_kernel).
// DYN: the XCD's workgroups take the items of its list from a counter (one
// atomic per tile) instead of every wx-th one; the host puts the problem
// with the most K blocks first.  With problems of very different K (dgrad
// over N next to wgrad over the token count) a fixed stride hands a few
// workgroups the long tiles on top of their share of short ones.
// AMAX: the epilogue also takes max |C| over the bf16 values it stores
// (rows < M, columns < N), so that the next layer's dynamic scaling needs
// no amax pass over C.  A workgroup keeps one running max while it walks
// one problem's tiles (its share of a problem is contiguous) and folds it
// into that problem's amax_out with one atomic max when it moves on to
// another problem or ends.
template <int FA, int FB, int BM, int BN, int WGM, int WGN, int MINB, int G, bool PARTIAL, bool DYN = false,
          bool AMAX = false, bool ODD = false>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_fp8_tn_kernel(const Batch batch) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA tiles per wave
  constexpr int OPA = BM * kBK, OPB = BN * kBK;  // bytes per operand per stage
  constexpr int STB = OPA + OPB;
  constexpr int LA = OPA / 1024 / NW, LB = OPB / 1024 / NW;  // 1 KB copies per wave per stage
  constexpr int LQ = LA + LB;
  constexpr int RB = WTN * 2;  // bytes per staged output row
  // 256 x 256 tiles with four waves take the K loop below that holds three
  // half-blocks of fragments in registers; the others two waves per SIMD
  constexpr bool kStag = BM == 256 && BN == 256 && NW == 4;
  static_assert(LA >= 1 && LB >= 1 && TM >= 1 && TN >= 2, "tile configuration");
  static_assert(!(DYN && PARTIAL), "split problems keep the fixed stride");
  static_assert(!(AMAX && PARTIAL), "split problems take their amax in the reduce kernel");
  static_assert(kStag || LQ <= 15, "vmcnt immediate");
  static_assert(NW * WTM * RB <= 2 * STB, "epilogue staging must fit in LDS");
  // two stages of A and B (the epilogue reuses them for its staging); DYN
  // also keeps its two next-item slots past them and AMAX one word per wave,
  // in the same array (a second __shared__ object makes the compiler wait
  // for the LDS copies before every fragment read)
  constexpr int kDynBytes = DYN ? 16 : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STB + kDynBytes + (AMAX ? 4 * 64 * NW : 0)];

  const int tid = threadIdx.x, lane = tid & 63;
  // (with 256 x 256 tiles the wave index is held as a scalar: a vector copy
  // would be spilled and reloaded at every tile)
  const int wave = kStag ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int g = lane >> 5;  // K half within a 64-byte sub-step
  const int wm = (wave / WGN) * WTM, wn = (wave % WGN) * WTN;

  // This workgroup's share of the tiles: XCD x owns a contiguous 1/8 of each
  // problem's tile list (so problems of different K stay balanced across
  // XCDs), and its wx workgroups take every wx-th tile of that share (DYN:
  // the first wx in order, the rest from the XCD's counter).
  const int xcd = (int)blockIdx.x % kXcds, local_wg = (int)blockIdx.x / kXcds;
  const int nwg = (int)gridDim.x;
  const int wx = nwg / kXcds + (xcd < nwg % kXcds ? 1 : 0);
  // start / length of this XCD's share of problem i (scalar arithmetic,
  // redone per tile rather than kept in registers across the K loop)
  auto share = [&](int i, int &start_i, int &len_i) {
    const int T = i < batch.count ? batch.p[i].tiles_m * batch.p[i].tiles_n * (PARTIAL ? batch.p[i].splits : 1) : 0;
    const int per = T / kXcds, rem = T % kXcds;
    start_i = xcd * per + min(xcd, rem);
    len_i = per + (xcd < rem ? 1 : 0);
  };
  int total = 0;
#pragma unroll
  for (int i = 0; i < kMaxGemms; ++i) {
    int st, ln;
    share(i, st, ln);
    total += ln;
  }

  // DYN: item wx + i goes to the workgroup whose fetch returned i.  Thread 0
  // fetches at the start of a tile and publishes the value in next_item[par]
  // once its tile's first copies are in; every thread reads it after the
  // tile's last barrier.  Two slots, alternating per tile: the write of a
  // slot and the previous read of it are always a barrier apart.  Every
  // thread issues the fetch, so that it sits under no branch: where a branch
  // joins, the compiler would wait for the result at once -- and, vmcnt
  // being in order, for the previous tile's output stores.  It is a buffer
  // atomic on the XCD's one-word counter, and only thread 0's offset lies
  // inside that range: the range check discards every other lane's add.
  // Issued before the tile's copies, it has returned once the prologue's
  // wait for block 0 does, so its use there costs no wait of its own.
  int *const next_item = reinterpret_cast<int *>(smem + 2 * STB);
  int par = 0;
  // AMAX: each lane's running max magnitude (15-bit bf16 field) of the
  // values problem amax_pi's tiles stored, in LDS (red[tid], updated by its
  // own lane after the tile's stores are issued: no register lives across the
  // K loop for it, and no cross-lane step runs per tile); flushed by a
  // workgroup max and one atomic.
  uint32_t *const red = reinterpret_cast<uint32_t *>(smem + 2 * STB + kDynBytes);
  int amax_pi = -1;
  if constexpr (AMAX) red[tid] = 0;  // only this lane touches red[tid] until a flush
  auto flush_amax = [&]() {
    if constexpr (AMAX) {
      uint32_t m = red[tid];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
      __syncthreads();  // every lane has read its word
      if (lane == 0) red[wave] = m;
      __syncthreads();
      if (tid == 0 && amax_pi >= 0 && batch.p[amax_pi].amax_out) {
#pragma unroll
        for (int w = 1; w < NW; ++w) m = max(m, red[w]);
        atomicMax(reinterpret_cast<uint32_t *>(batch.p[amax_pi].amax_out), m << 16);
      }
      __syncthreads();  // read before any lane clears its word
      red[tid] = 0;
    }
  };
  uint32_t *const queue = DYN ? batch.queue + xcd * kQueueWords : nullptr;
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void *)queue, (short)0, 4, 0x00020000);
  for (int it = local_wg; it < total;) {
    uint32_t fetched = 0;
    if constexpr (DYN) fetched = (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, qrs, tid == 0 ? 0 : kOutOfRange, 0, 0);
    auto publish = [&]() {
      if constexpr (DYN) {
        if (tid == 0) next_item[par] = (int)fetched + wx;
      }
    };
    // problem pi, tile t of it: this XCD's shares of the problems follow one another
    int pi = 0, off = it, t = 0;
#pragma unroll
    for (int i = 0; i < kMaxGemms; ++i) {
      int st, ln;
      share(i, st, ln);
      if (pi == i) {
        if (off >= ln && i + 1 < kMaxGemms) {
          off -= ln;
          pi = i + 1;
        } else {
          t = st + off;
        }
      }
    }
    if constexpr (AMAX) {
      if (pi != amax_pi) {  // uniform: the workgroup moves on to another problem
        if (amax_pi >= 0) flush_amax();
        amax_pi = pi;
      }
    }
    const Problem P = batch.p[pi];
    const int M = P.M, N = P.N;
    const int lda = P.lda, ldb = P.ldb;  // row strides of the operands
    // the K range this tile contracts: all of K, or its split's whole K blocks
    int K = P.K, kbase = 0, range = 0;
    if constexpr (PARTIAL) {
      const int per = P.tiles_m * P.tiles_n;
      range = t / per;
      t -= range * per;
      const int nkb = (P.K + kBK - 1) / kBK;
      const int kb0 = range * nkb / P.splits, kb1 = (range + 1) * nkb / P.splits;
      kbase = kb0 * kBK;
      K = min(kb1 * kBK, P.K) - kbase;
    }
    // The inverse scales through the scalar cache (the kernel never writes
    // them), read here so that the epilogue does not wait for them.
    typedef const __attribute__((address_space(4))) float cfloat;
    const float inv_a = *(cfloat *)P.inv_a, inv_b = *(cfloat *)P.inv_b;
    int tm, tn;
    tile_coords<G>(t, P.tiles_m, P.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    // (rows past the tile's last row lie outside the range; bytes past the
    // range's K are masked in issue_one)
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.a + (int64_t)m0 * lda + kbase), (short)0, rows_a * lda - kbase, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.b + (int64_t)n0 * ldb + kbase), (short)0, rows_b * ldb - kbase, 0x00020000);

    // Global offset (without the K block base) and K byte of each 16-byte
    // slot this lane copies: A slot s = (wave * LA + j) * 64 + lane, same for B.
    int offa[LA], kca[LA], offb[LB], kcb[LB];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int s = (wave * LA + j) * 64 + lane;
      const int r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
      offa[j] = r * lda + c * 16;
      kca[j] = c * 16;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int s = (wave * LB + j) * 64 + lane;
      const int r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
      offb[j] = r * ldb + c * 16;
      kcb[j] = c * 16;
    }
    // copy q (0 .. LQ-1) of K block kt into stage kt & 1
    // Tiles in odd bands of eight tile-columns walk K from the end (whole K
    // blocks only, so no ragged block moves): an XCD's tiles advance a patch
    // along a row band, and the patch that follows reads the same A rows
    // starting with the K blocks its predecessor read last, still in the L2.
    // The direction is a function of the tile alone, so a problem gives the
    // same bits in any launch or batch (measured, same box: the Llama-8B
    // layer's backward pairs 414.7 -> 402.5 us, its step 5195 -> 5088 us;
    // the 65536-row step 3043 -> 3017 us).
    const int nkb = (K + kBK - 1) / kBK;
    const bool rev = ((tn >> 3) & 1) && K % kBK == 0;
    auto issue_one = [&](int kt, int q) {
      const int k0 = (rev ? nkb - 1 - kt : kt) * kBK;
      uint8_t *stage = smem + (kt & 1) * STB;
      if (q < LA) {
        const int vo = (kca[q] + k0 < K) ? offa[q] + k0 : kOutOfRange;  // past K: outside the range -> 0
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void *)(stage + (wave * LA + q) * 1024), 16, vo, 0, 0, 0);
      } else {
        const int j = q - LA;
        const int vo = (kcb[j] + k0 < K) ? offb[j] + k0 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void *)(stage + OPA + (wave * LB + j) * 1024), 16, vo, 0,
                                                 0, 0);
      }
    };

    int arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) brow[j] = wn + j * 32 + (lane & 31);
    // Fragment of row r for sub-step ks (0/1) of the K block in `stage`:
    // chunks ks*4 + g*2 and +1 (32 K-bytes).
    auto rd = [&](int stage, int op_off, int r, int ks) {
      const u32x4 *st = (const u32x4 *)(smem + stage * STB + op_off);
      const int c = ks * 4 + g * 2;
      const u32x4 lo = st[slot128(r, c)], hi = st[slot128(r, c + 1)];
      return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // (256 x 256 tiles of four waves: 8 x 8 blocks of 16 x 16 instead)
    v4f acc4[kStag ? 8 : 1][kStag ? 8 : 1];
    if constexpr (kStag) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc4[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    auto mfma = [&](const v8i &a, const v8i &b, v16f &c) {
      c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
    };
    const int nk = (K + kBK - 1) / kBK;
    // A last K block with at most 64 bytes left (K = 1600, 4800) holds only
    // zeros in its second sub-step: those MFMAs would add exact zeros to
    // accumulators that can never be -0, so they are skipped (same bits).
    const bool tail_half = K - (nk - 1) * kBK <= kBK / 2;
    if constexpr (!kStag) {
      v8i fa[TM], fb[TN];
      auto col0 = [&]() {
#pragma unroll
        for (int i = 0; i < TM; ++i) mfma(fa[i], fb[0], acc[i][0]);
      };
      // Columns 1 .. TN-1 of the current sub-step.  With REFILL, fb[j] is
      // refilled with sub-step (stage, ks) after column j and fa[i] after its
      // MFMA in the last column (fb[0] was refilled by the caller); with
      // kt >= 0, the LQ copies of K block kt are spread over these MFMAs.
      auto cols = [&](auto REFILL, int stage, int ks, int kt) {
        constexpr int nmf = (TN - 1) * TM;
        int q = 0, mf = 0;
#pragma unroll
        for (int j = 1; j < TN; ++j) {
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            mfma(fa[i], fb[j], acc[i][j]);
            if constexpr (decltype(REFILL)::value) {
              if (j == TN - 1) fa[i] = rd(stage, 0, arow[i], ks);
            }
            ++mf;
            if (kt >= 0) {
              const int upto = (mf * LQ + nmf - 1) / nmf;
              while (q < upto) issue_one(kt, q++);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (decltype(REFILL)::value) fb[j] = rd(stage, OPA, brow[j], ks);
        }
      };
      // K block s: the fragments hold its sub-step 0 and column 0 is done.
      // NEXT: a block s+1 exists; DMA: block s+2 exists (copied during this one).
      auto block = [&](int s, auto NEXT, auto DMA) {
        const int cb = s & 1;
        __builtin_amdgcn_sched_barrier(0);
        fb[0] = rd(cb, OPA, brow[0], 1);
        cols(bool_t<true>(), cb, 1, -1);  // rest of sub-step 0; fragments <- sub-step 1
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(NEXT)::value) {
          col0();
          __builtin_amdgcn_sched_barrier(0);
          // block s+1 resident (own copies, then everyone's), every read of
          // block s done everywhere: its buffer can take block s+2
          __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          fb[0] = rd(cb ^ 1, OPA, brow[0], 0);
          cols(bool_t<true>(), cb ^ 1, 0, decltype(DMA)::value ? s + 2 : -1);
          __builtin_amdgcn_sched_barrier(0);
          col0();
        } else if (!tail_half) {
          col0();
          __builtin_amdgcn_sched_barrier(0);
          cols(bool_t<false>(), 0, 0, -1);
        }
      };

      if (nk > 0) {
#pragma unroll
        for (int q = 0; q < LQ; ++q) issue_one(0, q);
        if (nk > 1) {
#pragma unroll
          for (int q = 0; q < LQ; ++q) issue_one(1, q);
          __builtin_amdgcn_s_waitcnt(0x0F70 | LQ);  // vmcnt(LQ): block 0 resident
        } else {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
        __builtin_amdgcn_s_barrier();
        publish();
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = rd(0, OPA, brow[j], 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = rd(0, 0, arow[i], 0);
        col0();
        int s = 0;
        for (; s + 2 < nk; ++s) block(s, bool_t<true>(), bool_t<true>());
        if (s + 1 < nk) block(s++, bool_t<true>(), bool_t<false>());
        block(s, bool_t<false>(), bool_t<false>());
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the fetch has returned
        publish();
      }
    } else {
      // Four waves of 128 x 128 (one per SIMD), v_mfma_f32_16x16x128_f8f6f4
      // on C^T: 8 x 8 accumulator blocks of 16 x 16, and a fragment is 16
      // rows of one operand over a whole K block.  Lane l holds row l & 15,
      // 16-byte chunks q and q + 4 of the block (q = l >> 4): A and B take
      // the same K bytes per lane, so any such split gives the product, and
      // this one keeps the fragment reads free of LDS bank conflicts
      // (chunks 2q and 2q + 1 cost an extra cycle per read: ~32k conflict
      // cycles per tile in SQ_LDS_BANK_CONFLICT).  Per flop the instruction
      // moves half the accumulator data of the 32 x 32 x 64 one; on random
      // codes the chip then holds a ~8% higher clock.  A region is one
      // operand of one K block: region 2 kb + X (X = 0: A, 1: B);
      // consecutive blocks alternate between the two stages.
      // Step j = 2 s + h runs 32 MFMAs of K block s from registers: A
      // fragments 4h .. 4h + 3 against all eight B fragments (h = 0: A
      // fragment by fragment; h = 1: B fragment by fragment).  Meanwhile it
      // reads all fragments of region j + 2 (one operand of block s + 1) and
      // copies region j + 5 over region j + 1, which step j - 1 finished
      // reading.  So every step issues the same share of copies, and a copy
      // has two to three steps to land before its region is read.  A
      // fragment of block s + 1 is mostly read right after the fragment of
      // block s it replaces has had its last MFMA, so at most ~22 fragments
      // are live.  The barrier of step j sits after its fourth MFMA: each
      // wave has then finished the reads of step j - 1 and received all its
      // copies of region j + 2.
      static_assert(TM == 4 && TN == 4 && LA == 8 && LB == 8 && OPA == OPB, "four 128 x 128 wave tiles");
      // The sequence of steps is fixed by the parity of the count of K
      // blocks: ODD launches (every problem's count odd) end with a nine-step
      // tail, the others with a seven-step one.  In the latter an odd count
      // gets a virtual block at the end, so that one sequence of steps serves
      // with no branch: its copies fetch zeros, and its two steps (MFMAs
      // only) add exact zeros to accumulators that can never hold -0 (same
      // bits).
      const int virt = ODD ? 0 : nkb & 1, nkp = nkb + virt;
      const int swave = wave;  // (a scalar here)
      // lane-derived addresses are computed per tile from a regenerated lane
      // index (kept across the tile loop they would be spilled, and a spill
      // reload waits for every copy and store in flight)
      const int kl = lane_here();
      // Layout: A of stages 0 and 1, then B of stages 0 and 1, so that every
      // fragment read of one operand is a lane base plus an immediate offset
      // below 64 KB (four bases per operand).
      auto region = [&](int S, int X) { return smem + X * 2 * OPA + S * OPA; };
      // Byte offset, within a region, of this lane's 16-byte chunk lo (0/1)
      // in fragment 0 of operand X: row r = w + l (w the wave's first row, a
      // multiple of 16; l = lane & 15), chunk c = (lane >> 4) + 4 lo, at
      // slot128(r, c); fragment f is 16 rows (2048 bytes) on.
      int rdb[2][2];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int lo = 0; lo < 2; ++lo) {
          const int l = kl & 15, c = (kl >> 4) + 4 * lo;
          rdb[X][lo] = ((X ? wn : wm) + l) * 128 + ((c ^ ((l >> 1) & 7)) << 4);
        }
      auto rd16 = [&](int S, int X, int f) {
        const uint8_t *st = region(S, X) + f * 2048;
        const u32x4 lo = *(const u32x4 *)(st + rdb[X][0]), hi = *(const u32x4 *)(st + rdb[X][1]);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      v8i fa[2][8], fb[2][8];  // [block parity][fragment]
      // Copy q's slots (LA = 8) start 16 (q >> 1) rows past those of copy
      // q & 1: its global offset is one of two per-lane bases plus a uniform
      // row step, and its K byte the base's chunk.
      int cbase_a[2], cbase_b[2], kc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = swave * 64 + (kl >> 3) + 8 * e;
        kc[e] = 16 * ((kl & 7) ^ (kl >> 4) ^ (e << 2));
        cbase_a[e] = r * lda + kc[e];
        cbase_b[e] = r * ldb + kc[e];
      }
      // K block order: with a ragged K the ragged (physical last) block goes
      // first, so that only the prologue's copies need a per-lane K mask;
      // otherwise forward, or from the end on odd tile bands (above).
      const bool ragged = K % kBK != 0;
      // Copy q of region (X, pipeline block kb) into stage S.  The row stays
      // in the per-lane offset (rows past the tile fail the range check) and
      // the block's K offset rides in the scalar offset.  MODE 0: a whole
      // block; 2: the last pipeline block (all lanes out of range when it is
      // the virtual one, which loads zeros); 1: a block of the prologue, which
      // may be the ragged one (lanes whose 16 bytes start at or past K out of
      // range: K is a multiple of 16).
      // The K byte offset of pipeline block kb >= 1 is linear in kb (kept in
      // scalar registers): forward from -ragged blocks, or backward from nkb - 1
      // (odd tile bands); clamped to the whole blocks for the virtual one.
      const int kstep = __builtin_amdgcn_readfirstlane(rev ? -kBK : kBK);
      const int k00 = __builtin_amdgcn_readfirstlane(rev ? (nkb - 1) * kBK : (ragged ? -kBK : 0));
      const int kmax = __builtin_amdgcn_readfirstlane((nkb - 1 - (ragged ? 1 : 0)) * kBK);
      // row steps of the copies (16 rows per pair of copies), scalar
      const int rstep_a = __builtin_amdgcn_readfirstlane(16 * lda), rstep_b = __builtin_amdgcn_readfirstlane(16 * ldb);
      auto copy_region = [&](auto X_, auto S_, auto MODE_, int kb, int q) {
        constexpr int X = decltype(X_)::value, S = decltype(S_)::value, MODE = decltype(MODE_)::value;
        lds_void *dst = (lds_void *)(region(S, X) + (swave * LA + q) * 1024);
        // Row offset: the lane's base plus a multiple of the scalar row step,
        // added by an opaque instruction so that the compiler does not hold
        // all sixteen offsets in registers across the K loop.
        int vrow = X == 0 ? cbase_a[q & 1] : cbase_b[q & 1];
        if ((q >> 1) > 0) {  // (q is known after unrolling)
          const int st = (q >> 1) * (X == 0 ? rstep_a : rstep_b);
          asm volatile("v_add_u32 %0, %1, %2" : "=v"(vrow) : "s"(st), "v"(vrow));
        }
        if constexpr (MODE == 0) {
          const int k0 = min(max(k00 + kb * kstep, 0), kmax);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(X == 0 ? rsa : rsb, dst, 16, vrow, k0, 0, 0);
        } else if constexpr (MODE == 2) {
          const int k0 = min(max(k00 + kb * kstep, 0), kmax);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(X == 0 ? rsa : rsb, dst, 16, virt ? kOutOfRange : vrow, k0, 0, 0);
        } else {
          const int kp = rev ? nkb - 1 - kb : (ragged ? (kb == 0 ? nkb - 1 : kb - 1) : kb);
          const int k0 = kp * kBK;
          const int vo = kc[q & 1] + k0 < K ? vrow : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(X == 0 ? rsa : rsb, dst, 16, vo, __builtin_amdgcn_readfirstlane(k0),
                                                   0, 0);
        }
      };
      auto copy_all = [&](auto X_, auto S_, int kb) {
#pragma unroll
        for (int q = 0; q < LA; ++q) copy_region(X_, S_, int_t<1>(), kb, q);
      };
      // The fragment read and the copy issued after each MFMA slot of a step
      // (all after the barrier at slot 3).  A step (h = 0): the next block's
      // A fragments 4-7 at once, then 0-3 as the current fragments 0, 1, 2
      // have their last MFMAs (slots 7, 15, 23).  B step (h = 1): next
      // fragment f after the current one's last MFMA (slot 4 f + 3), 5-7 a
      // little early, so that the last read is eight MFMAs ahead of its use.
      constexpr int kRdA[32] = {-1, -1, -1, -1, 4,  5,  6,  7,  0,  -1, -1, -1, 1,  -1, -1, -1,
                                2,  -1, -1, -1, 3,  -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
      constexpr int kRdB[32] = {-1, -1, -1, -1, 0,  -1, -1, -1, 1,  -1, -1, -1, 2,  -1, -1, -1,
                                3,  -1, -1, -1, 4,  -1, 5,  6,  7,  -1, -1, -1, -1, -1, -1, -1};
      constexpr int kCp[32] = {-1, -1, -1, -1, -1, -1, 0,  -1, -1, 1,  -1, -1, -1, 2,  -1, -1,
                               -1, 3,  -1, -1, -1, 4,  -1, -1, -1, 5,  -1, 6,  -1, 7,  -1, -1};
      auto mfma16 = [&](const v8i &a, const v8i &b, v4f &c) {
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, FB, FA, 0, 0, 0, 0);
      };
      // step j (block parity P, half H); RD / CP: whether region j + 2 / j + 5
      // exist; MODE: the copies' kind; VM: copies of this wave that may still
      // be in flight at the barrier (those of regions j + 3 and j + 4 that
      // exist); BAR: whether the step needs the barrier at all (the last two
      // do not)
      auto step = [&](auto P_, auto H_, auto RD, auto CP, auto MODE, auto BAR, int vm, int j) {
        constexpr int P = decltype(P_)::value, H = decltype(H_)::value;
        constexpr int RP = P ^ 1, CS = H == 0 ? P : P ^ 1;
        const int ckb = (j + 5) >> 1;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          {
            const int i = H == 0 ? t >> 3 : 4 + (t & 3), jj = H == 0 ? t & 7 : t >> 2;
            mfma16(fa[P][i], fb[P][jj], acc4[i][jj]);
          }
          if (t == 3 && BAR) {
            if (vm >= 16)
              __builtin_amdgcn_s_waitcnt(0x4070);  // vmcnt(16) lgkmcnt(0)
            else if (vm >= 8)
              __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8) lgkmcnt(0)
            else
              __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
          }
          if constexpr (H == 0) {
            if (RD && kRdA[t] >= 0) fa[RP][kRdA[t]] = rd16(RP, 0, kRdA[t]);
          } else {
            if (RD && kRdB[t] >= 0) fb[RP][kRdB[t]] = rd16(RP, 1, kRdB[t]);
          }
          if (CP && kCp[t] >= 0) copy_region(int_t<H ^ 1>(), int_t<CS>(), MODE, ckb, kCp[t]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      const auto T = bool_t<true>();
      auto full = [&](auto P_, auto H_, int j) { step(P_, H_, T, T, int_t<0>(), T, 16, j); };
      // A step d steps before the last one (d <= 6): it reads region j + 2
      // while d >= 2, copies region j + 5 (the last block's) while d >= 5,
      // and may leave in flight the copies of the regions after j + 2 that
      // exist (two while d >= 4, one at d = 3).
      auto tstep = [&](auto D_, auto P_, auto H_, int j) {
        constexpr int d = decltype(D_)::value;
        if constexpr (d >= 2) {
          step(P_, H_, T, bool_t<(d >= 5)>(), int_t<2>(), T, d >= 4 ? 16 : (d == 3 ? 8 : 0), j);
        } else {
          // the last block: MFMAs only
          step(P_, H_, bool_t<false>(), bool_t<false>(), int_t<0>(), bool_t<false>(), 0, j);
        }
      };
      // steps j .. j + D0 (d = D0 .. 0), the first of parity (P0, H0)
      auto tail = [&](auto D0_, auto P0_, auto H0_, int j) {
        constexpr int D0 = decltype(D0_)::value, p0 = decltype(P0_)::value, h0 = decltype(H0_)::value;
        static_assert(D0 <= 8, "tail length");
        tstep(int_t<D0>(), int_t<p0>(), int_t<h0>(), j);
        if constexpr (D0 >= 1) tstep(int_t<D0 - 1>(), int_t<step_p(p0, h0, 1)>(), int_t<(h0 + 1) & 1>(), j + 1);
        if constexpr (D0 >= 2) tstep(int_t<D0 - 2>(), int_t<step_p(p0, h0, 2)>(), int_t<(h0 + 2) & 1>(), j + 2);
        if constexpr (D0 >= 3) tstep(int_t<D0 - 3>(), int_t<step_p(p0, h0, 3)>(), int_t<(h0 + 3) & 1>(), j + 3);
        if constexpr (D0 >= 4) tstep(int_t<D0 - 4>(), int_t<step_p(p0, h0, 4)>(), int_t<(h0 + 4) & 1>(), j + 4);
        if constexpr (D0 >= 5) tstep(int_t<D0 - 5>(), int_t<step_p(p0, h0, 5)>(), int_t<(h0 + 5) & 1>(), j + 5);
        if constexpr (D0 >= 6) tstep(int_t<D0 - 6>(), int_t<step_p(p0, h0, 6)>(), int_t<(h0 + 6) & 1>(), j + 6);
        if constexpr (D0 >= 7) tstep(int_t<D0 - 7>(), int_t<step_p(p0, h0, 7)>(), int_t<(h0 + 7) & 1>(), j + 7);
        if constexpr (D0 >= 8) tstep(int_t<D0 - 8>(), int_t<step_p(p0, h0, 8)>(), int_t<(h0 + 8) & 1>(), j + 8);
      };

      // (the host sends only problems of at least four K blocks here)
      // Prologue: blocks 0 and 1 copied, block 0 read whole, then region 4
      // (block 2's A) copied over block 0's A.  Block i sits in stage i & 1.
      copy_all(int_t<0>(), int_t<0>(), 0);
      copy_all(int_t<1>(), int_t<0>(), 0);
      copy_all(int_t<0>(), int_t<1>(), 1);
      copy_all(int_t<1>(), int_t<1>(), 1);
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): block 0 resident
      __builtin_amdgcn_s_barrier();
      publish();
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        fa[0][f] = rd16(0, 0, f);
        fb[0][f] = rd16(0, 1, f);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): block 0 read by this wave
      __builtin_amdgcn_s_barrier();         // ... and by all
      copy_all(int_t<0>(), int_t<0>(), 2);
      full(int_t<0>(), int_t<0>(), 0);
      // 2 nkp steps: step 0, rounds of four, and the tail (its first step
      // always of parity (0, 1))
      constexpr int kTail = ODD ? 8 : 6;
      int j = 1;
      if (nkp > (ODD ? 5 : 4)) {
        // (the loop's first round peeled: the register allocator then keeps
        // the fragments where the loop wants them)
        full(int_t<0>(), int_t<1>(), 1);
        full(int_t<1>(), int_t<0>(), 2);
        full(int_t<1>(), int_t<1>(), 3);
        full(int_t<0>(), int_t<0>(), 4);
        for (j = 5; j + 4 <= 2 * nkp - 1 - kTail; j += 4) {
          full(int_t<0>(), int_t<1>(), j);
          full(int_t<1>(), int_t<0>(), j + 1);
          full(int_t<1>(), int_t<1>(), j + 2);
          full(int_t<0>(), int_t<0>(), j + 3);
        }
      }
      tail(int_t<kTail>(), int_t<0>(), int_t<1>(), j);
    }

    if constexpr (PARTIAL) {
      const int rows_c = min(BM, M - m0);
      const __amdgpu_buffer_rsrc_t rsp = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(reinterpret_cast<float *>(P.c) + ((int64_t)range * M + m0) * N), (short)0, rows_c * N * 4,
          0x00020000);
      // (the lane index regenerated here with the four-wave tiles: the
      // addresses are derived per tile, not kept across the K loop)
      const int pl = kStag ? lane_here() : lane;
      if constexpr (kStag) {
        // fp32 partial product, unscaled: lane (row r = lane & 15, quarter q
        // = lane >> 4) holds columns 4q .. 4q + 3 of row r of each 16 x 16
        // block (the MFMA ran on C^T): one 16-byte store each; rows past M
        // lie outside the slab's range, columns past N get an offset outside
        // it.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = wm + i * 16 + (pl & 15);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int col = n0 + wn + j * 16 + 4 * (pl >> 4);
            const int vo = col < N ? (row * N + col) * 4 : kOutOfRange;
            const u32x4 v{__float_as_uint(acc4[i][j][0]), __float_as_uint(acc4[i][j][1]),
                          __float_as_uint(acc4[i][j][2]), __float_as_uint(acc4[i][j][3])};
            __builtin_amdgcn_raw_buffer_store_b128(v, rsp, vo, 0, 0);
          }
        }
      } else {
        // lane (column c = lane & 31, half h) holds rows 8*(v>>2) + 4*h +
        // (v&3) of each 32x32 tile; 32 lanes write 128 contiguous bytes of a
        // row
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn + j * 32 + (pl & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int row = wm + i * 32 + 8 * (v >> 2) + 4 * (pl >> 5) + (v & 3);
              const int vo = col < N ? (row * N + col) * 4 : kOutOfRange;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rsp, vo, 0, 0);
            }
          }
      }
      __syncthreads();  // every wave is done with the stage buffers before the next tile's copies
      it += wx;
      continue;
    }

    // Epilogue: the tile, scaled (+ bias) and rounded to bf16, is staged in
    // LDS row by row per wave, then read back in 16-byte row chunks and
    // stored.
    __syncthreads();  // every wave is done with the stage buffers
    const float alpha = inv_a * inv_b;
    // The lane index of the epilogue: with 256 x 256 tiles regenerated here,
    // so that the compiler derives the epilogue's addresses from it per tile
    // instead of keeping them (spilled) across the K loop.
    const int el = kStag ? lane_here() : lane;
    uint8_t *wreg = smem + wave * (WTM * RB);
    // Staged row r, 16-byte chunk ch: at wreg + r * RB + chunk_at(r, ch).
    //  * 256 x 256 tiles (RB = 256, one full set of banks): the MFMA ran on
    //    C^T, so lane (row r = lane & 15 of each 16 x 16 block (i, j),
    //    quarter q = lane >> 4) holds columns 4q .. 4q + 3 of row r: 8 bytes
    //    of bf16, half q & 1 of chunk 2j + (q >> 1).  Chunks are XOR-ed with
    //    r, so the 32 lanes of either half of a wave write 32 distinct 8-byte
    //    slots of the 256 banks' row.
    //  * smaller tiles (RB = 128): lane (column c = lane & 31, half h) holds
    //    rows 8*(v>>2) + 4*h + (v&3) for v = 0..15.  Even lanes take column
    //    pair (c, c+1) at even v, odd lanes (c-1, c) at odd v: each lane keeps
    //    one of its values v = 2k, 2k+1 and sends the other to the neighbour
    //    lane (a DPP swap folded into the scaling multiply); the pair, rounded
    //    to bf16 as (kept, received), is one 32-bit LDS word, its halves
    //    swapped on odd lanes (a rotate by a per-lane amount).  Rows of even /
    //    odd v differ in parity and rows of the two halves in bit 2 (which
    //    swaps the 64-byte halves of the row), so each write is free of bank
    //    conflicts.
    auto chunk_at = [](int row, int ch) {
      return kStag ? ((ch ^ (row & 15)) << 4) : ((ch * 16) ^ (((row >> 2) & 1) << 6));
    };
    if constexpr (kStag) {
      static_assert(RB == 256, "staging of the 256 x 256 tiles");
      const int r = el & 15, q = el >> 4;
      auto stage_t = [&](auto BIAS) {
        // bias of this lane's four columns of each block column j (bf16
        // words), all eight loads issued before the first use: through a
        // range-checked buffer, columns at or past N read zeros with no
        // branch, so the loads share one wait
        u32x2 bws[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bws[j] = u32x2{0u, 0u};
        if constexpr (decltype(BIAS)::value) {
          const __amdgpu_buffer_rsrc_t rbias =
              __builtin_amdgcn_make_buffer_rsrc((void *)P.bias, (short)0, N * 2, 0x00020000);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            bws[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rbias, (n0 + wn + j * 16 + 4 * q) * 2, 0, 0));
          __builtin_amdgcn_sched_barrier(0);  // (kept ahead of the scaling)
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2 bw = bws[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = i * 16 + r;
            float x0 = acc4[i][j][0] * alpha, x1 = acc4[i][j][1] * alpha;
            float x2 = acc4[i][j][2] * alpha, x3 = acc4[i][j][3] * alpha;
            if constexpr (decltype(BIAS)::value) {
              x0 += __uint_as_float(bw.x << 16);
              x1 += __uint_as_float(bw.x & 0xFFFF0000u);
              x2 += __uint_as_float(bw.y << 16);
              x3 += __uint_as_float(bw.y & 0xFFFF0000u);
            }
            const u32x2 w{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2)),
                          __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x2, x3}, bf16x2))};
            *(u32x2 *)(wreg + row * RB + chunk_at(row, 2 * j + (q >> 1)) + 8 * (q & 1)) = w;
          }
        }
      };
      if (P.bias)
        stage_t(bool_t<true>());
      else
        stage_t(bool_t<false>());
    } else {
      const bool odd = el & 1;
      const uint32_t rot = odd ? 16u : 0u;
      auto stage_out = [&](auto BIAS) {
        // bias of the kept and the received value of this lane's column pair
        // (cpair, cpair + 1) of each 32-column tile j
        // (a range-checked buffer: columns at or past N read zeros, no branch)
        float bias_keep[TN], bias_recv[TN];
        const __amdgpu_buffer_rsrc_t rbias =
            __builtin_amdgcn_make_buffer_rsrc((void *)P.bias, (short)0, N * 2, 0x00020000);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          bias_keep[j] = bias_recv[j] = 0.0f;
          if constexpr (decltype(BIAS)::value) {
            const uint32_t bw = __builtin_amdgcn_raw_buffer_load_b32(rbias, (n0 + wn + j * 32 + (el & 30)) * 2, 0, 0);
            const float lo = __uint_as_float(bw << 16), hi = __uint_as_float(bw & 0xFFFF0000u);
            bias_keep[j] = odd ? hi : lo;
            bias_recv[j] = odd ? lo : hi;
          }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cpair = j * 32 + (el & 30);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float a0 = acc[i][j][2 * k], a1 = acc[i][j][2 * k + 1];
              const float keep = odd ? a1 : a0, send = odd ? a0 : a1;
              const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, true));
              float ks = keep * alpha, rs = recv * alpha;
              if constexpr (decltype(BIAS)::value) {
                ks += bias_keep[j];
                rs += bias_recv[j];
              }
              const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{ks, rs}, bf16x2));
              const int v = 2 * k + (odd ? 1 : 0);
              const int row = i * 32 + 8 * (v >> 2) + 4 * (el >> 5) + (v & 3);
              *(uint32_t *)(wreg + row * RB + ((cpair * 2) ^ (((row >> 2) & 1) << 6))) =
                  __builtin_amdgcn_alignbit(w, w, rot);
            }
          }
      };
      if (P.bias)
        stage_out(bool_t<true>());
      else
        stage_out(bool_t<false>());
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // All of the wave's staged chunks are read first, then stored with
    // buffer stores: rows past M lie outside the tile's buffer range and
    // columns past N get an offset outside it, so no store needs a branch.
    constexpr int CPR = RB / 16;  // 16-byte chunks per row
    constexpr int NCH = WTM * CPR / 64;
    const int rows_c = min(BM, M - m0);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(P.c + (int64_t)m0 * N), (short)0, (int)((uint32_t)rows_c * (uint32_t)N * 2u), 0x00020000);
    // (in passes of at most 16 chunks per lane, to bound the registers held)
    constexpr int PASS = NCH < 16 ? NCH : 16;
    static_assert(NCH % PASS == 0, "epilogue passes");
    // AMAX: this lane's max magnitude of the values it stores, per 16-bit
    // half (both halves of a word compared at once by one packed max)
    u16x2 omag2 = u16x2{0, 0};
#pragma unroll
    for (int k0 = 0; k0 < NCH; k0 += PASS) {
      u32x4 vals[PASS];
      int offs[PASS];
#pragma unroll
      for (int u = 0; u < PASS; ++u) {
        const int idx = (k0 + u) * 64 + el;
        const int row = idx / CPR, ch = idx % CPR;
        vals[u] = *(const u32x4 *)(wreg + row * RB + chunk_at(row, ch));
        const int gcol = n0 + wn + ch * 8;
        offs[u] = gcol < N ? ((wm + row) * N + gcol) * 2 : kOutOfRange;
        if constexpr (AMAX) {
          // the values this chunk stores (padding rows may hold the bias: they
          // do not count): a mask, not a branch, drops the others
          const uint32_t keep = (gcol < N && wm + row < rows_c) ? 0x7FFF7FFFu : 0u;
          omag2 = __builtin_elementwise_max(omag2, __builtin_bit_cast(u16x2, vals[u].x & keep));
          omag2 = __builtin_elementwise_max(omag2, __builtin_bit_cast(u16x2, vals[u].y & keep));
          omag2 = __builtin_elementwise_max(omag2, __builtin_bit_cast(u16x2, vals[u].z & keep));
          omag2 = __builtin_elementwise_max(omag2, __builtin_bit_cast(u16x2, vals[u].w & keep));
        }
      }
      if (batch.nt_stores) {
#pragma unroll
        for (int u = 0; u < PASS; ++u) __builtin_amdgcn_raw_buffer_store_b128(vals[u], rsc, offs[u], 0, 2);  // nt
      } else {
#pragma unroll
        for (int u = 0; u < PASS; ++u) __builtin_amdgcn_raw_buffer_store_b128(vals[u], rsc, offs[u], 0, 0);
      }
    }
    if constexpr (AMAX)  // after the stores are issued
      red[tid] = max(red[tid], max((uint32_t)omag2.x, (uint32_t)omag2.y));
    __syncthreads();  // staging reads done before the next tile's copies land
    if constexpr (DYN) {
      it = __builtin_amdgcn_readfirstlane(next_item[par]);
      par ^= 1;
    } else {
      it += wx;
    }
  }
  if constexpr (AMAX) flush_amax();
  if constexpr (DYN) {
    // The last of the XCD's workgroups to get here clears its queue words.
    // Each workgroup's fetches have all returned (the last one ended its
    // loop) before it takes this ticket, so none can follow the clear.
    if (tid == 0 && atomicAdd(queue + 1, 1u) == (uint32_t)wx - 1) {
      atomicExch(queue, 0u);
      atomicExch(queue + 1, 0u);
    }
  }
}

// Skinny problems (M <= 64: the forward and dgrad of a handful of tokens)
// are bound by reading B once (N x K bytes) at HBM speed; the tiled kernel
// above would give them only N / 128 workgroups.  Here one workgroup of four
// waves owns 16 rows of B (16 output columns), so N / 16 workgroups stream
// B; the waves split K in 128-byte blocks (wave w takes blocks w, w + 4, ...),
// load both operands straight into registers, U blocks in flight per wave,
// and run v_mfma_f32_16x16x128_f8f6f4 once per 16-row block of A (lane l
// feeds row l % 16 and K bytes 32 * (l / 16) .. +32 of both operands; the
// accumulator of lane l holds rows 4 * (l / 16) + i, column l % 16).  The
// four waves' partial sums meet in LDS.
template <int FA, int FB, int MT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const Problem P) {
  constexpr int U = MT <= 2 ? 8 : 4;
  typedef float v4f_t __attribute__((ext_vector_type(4)));
  __shared__ v4f_t red[4][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (int)blockIdx.x * 16;
  const int M = P.M, N = P.N, K = P.K;
  const int rows_b = min(16, N - n0);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)P.a, (short)0, M * P.lda, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void *)(P.b + (int64_t)n0 * P.ldb), (short)0,
                                                                       rows_b * P.ldb, 0x00020000);
  const int r = lane & 15, kq = (lane >> 4) * 32;
  const int nkb = (K + kBK - 1) / kBK;
  v4f_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = v4f_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto load = [&](__amdgpu_buffer_rsrc_t rs, int ld, int row, int kb, int k) {
    // 32 bytes of `row` (stride ld) at K offset k of block kb; chunks past K
    // (or blocks past the end) point outside the range and read as zeros
    const int k0 = kb * kBK + k;
    const int o0 = (kb < nkb && k0 < K) ? row * ld + k0 : kOutOfRange;
    const int o1 = (kb < nkb && k0 + 16 < K) ? row * ld + k0 + 16 : kOutOfRange;
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o0, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o1, 0, 0));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  for (int kb0 = wave; kb0 < nkb; kb0 += 4 * U) {
    v8i fb[U], fa[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fb[u] = load(rsb, P.ldb, r, kb0 + 4 * u, kq);
#pragma unroll
      for (int m = 0; m < MT; ++m) fa[u][m] = load(rsa, P.lda, m * 16 + r, kb0 + 4 * u, kq);
    }
    __builtin_amdgcn_sched_barrier(0);  // all U blocks in flight before the first MFMA
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[u][m], fb[u], acc[m], FA, FB, 0, 0, 0, 0);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave == 0) {
    const float alpha = P.inv_a[0] * P.inv_b[0];
    uint32_t omag = 0;  // max magnitude of the stored values (for amax_out)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const v4f_t t = red[0][m][lane] + red[1][m][lane] + red[2][m][lane] + red[3][m][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + 4 * (lane >> 4) + i, col = n0 + (lane & 15);
        const float bv = P.bias ? __uint_as_float((uint32_t)P.bias[col < N ? col : 0] << 16) : 0.0f;
        const uint32_t h = f32_to_bf16_rne(t[i] * alpha + bv);
        if (row < M && col < N) {
          P.c[(int64_t)row * N + col] = (uint16_t)h;
          omag = max(omag, h & 0x7FFFu);
        }
      }
    }
    if (P.amax_out) {  // one atomic max per workgroup
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) omag = max(omag, (uint32_t)__shfl_xor((int)omag, off, 64));
      if (lane == 0) atomicMax(reinterpret_cast<uint32_t *>(P.amax_out), omag << 16);
    }
  }
}

constexpr int kSkinnyMaxM = 64;

template <int FA, int FB>
void launch_skinny(const Problem &p, hipStream_t stream) {
  const unsigned grid = (unsigned)((p.N + 15) / 16);
  switch ((p.M + 15) / 16) {
    case 1: gemm_skinny_kernel<FA, FB, 1><<<grid, 256, 0, stream>>>(p); break;
    case 2: gemm_skinny_kernel<FA, FB, 2><<<grid, 256, 0, stream>>>(p); break;
    case 3: gemm_skinny_kernel<FA, FB, 3><<<grid, 256, 0, stream>>>(p); break;
    default: gemm_skinny_kernel<FA, FB, 4><<<grid, 256, 0, stream>>>(p); break;
  }
}

// C = bf16(alpha * (sum over ranges of the fp32 partials, in range order)),
// the same fp32 scaling and rounding as the tiled kernel's epilogue; four
// elements per thread per step of a grid-stride loop (M * N is a multiple of
// 16).  amax_out (or null): max |C| folded in with one atomic per workgroup.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ part, int splits, int64_t mn,
                                                           const float *inv_a, const float *inv_b,
                                                           uint16_t *__restrict__ c, float *amax_out) {
  __shared__ uint32_t red[4];
  const float alpha = inv_a[0] * inv_b[0];
  uint32_t omag = 0;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += (int64_t)gridDim.x * 1024) {
    float4 acc = *reinterpret_cast<const float4 *>(part + i);
    for (int r = 1; r < splits; ++r) {
      const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)r * mn + i);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const bf16x2 lo = __builtin_convertvector(f32x2{acc.x * alpha, acc.y * alpha}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(f32x2{acc.z * alpha, acc.w * alpha}, bf16x2);
    const uint32_t wlo = __builtin_bit_cast(uint32_t, lo), whi = __builtin_bit_cast(uint32_t, hi);
    *reinterpret_cast<u32x2 *>(c + i) = u32x2{wlo, whi};
    omag = mag_max2(mag_max2(omag, wlo), whi);
  }
  if (amax_out) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) omag = max(omag, (uint32_t)__shfl_xor((int)omag, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = omag;
    __syncthreads();
    if (threadIdx.x == 0)
      atomicMax(reinterpret_cast<uint32_t *>(amax_out), max(max(red[0], red[1]), max(red[2], red[3])) << 16);
  }
}

// The tiled kernel with or without the output amax (only the forward's and
// dgrad's format pairs produce a tensor a next layer casts); four-wave
// 256 x 256 launches in fixed order whose problems all have an odd count of
// K blocks take the instantiation with the odd-count tail.
template <int FA, int FB, int BM, int BN, int WGM, int WGN, int MINB, int G, bool DYN>
void launch_tiled(const Batch &b, unsigned grid, bool amax, hipStream_t stream) {
  constexpr bool kAmaxPair = FB == 0;
  constexpr bool kOddTail = BM == 256 && BN == 256 && WGM * WGN == 4 && !DYN;
  if constexpr (kOddTail) {
    bool odd = true;
    for (int i = 0; i < b.count; ++i) odd &= ((b.p[i].K + kBK - 1) / kBK) % 2 == 1;
    if (odd) {
      if (kAmaxPair && amax)
        gemm_fp8_tn_kernel<FA, FB, BM, BN, WGM, WGN, MINB, G, false, DYN, kAmaxPair, true>
            <<<grid, 64 * WGM * WGN, 0, stream>>>(b);
      else
        gemm_fp8_tn_kernel<FA, FB, BM, BN, WGM, WGN, MINB, G, false, DYN, false, true>
            <<<grid, 64 * WGM * WGN, 0, stream>>>(b);
      return;
    }
  }
  if (kAmaxPair && amax)
    gemm_fp8_tn_kernel<FA, FB, BM, BN, WGM, WGN, MINB, G, false, DYN, kAmaxPair>
        <<<grid, 64 * WGM * WGN, 0, stream>>>(b);
  else
    gemm_fp8_tn_kernel<FA, FB, BM, BN, WGM, WGN, MINB, G, false, DYN><<<grid, 64 * WGM * WGN, 0, stream>>>(b);
}

// Whether the fixed tile stride leaves a batch of big tiles unbalanced: the
// kernel's walk (each XCD's share of every problem in turn; workgroup j of an
// XCD's wx takes items j, j + wx, ...) with each tile costing its K blocks
// plus ~6 blocks of prologue and epilogue, against an even split of the
// XCD's work.  Balanced batches keep the fixed stride: the work queue's
// per-tile fetch costs ~4% at 65536 x 4096 x 4096 (dX over 32 K blocks,
// dW over 512: each workgroup gets 16 of one and 1 of the other either way).
bool fixed_stride_unbalanced(const Batch &b, int nwg) {
  constexpr int kTileOverheadBlocks = 6;
  int64_t worst = 0, total = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int wx = nwg / kXcds + (x < nwg % kXcds ? 1 : 0);
    if (wx == 0) continue;
    std::vector<int64_t> load(wx, 0);
    int64_t item = 0;
    for (int i = 0; i < b.count; ++i) {
      const int T = b.p[i].tiles_m * b.p[i].tiles_n;
      const int len = T / kXcds + (x < T % kXcds ? 1 : 0);
      const int64_t cost = (b.p[i].K + kBK - 1) / kBK + kTileOverheadBlocks;
      for (int t = 0; t < len; ++t, ++item) load[item % wx] += cost;
    }
    for (int j = 0; j < wx; ++j) {
      worst = std::max(worst, load[j] * (int64_t)nwg);
      total += load[j];
    }
  }
  // worst workgroup more than 3% above the mean
  return worst * 100 > total * 103;
}

template <int FA, int FB>
void launch_fmt(Batch &b, float *split_ws, size_t split_bytes, uint32_t *queue, hipStream_t stream) {
  // skinny problems get their own launches; problems with few long tiles are
  // split along K when there is room for their partials; the rest share one
  // (problems of fewer than four K blocks, which the four-wave 256 x 256
  // kernel's pipeline does not take, go to a launch of their own)
  Batch rest{}, split{}, short_k{};
  const Problem *orig[kMaxGemms];
  size_t used = 0;
  for (int i = 0; i < b.count; ++i) {
    Problem &p = b.p[i];
    const int s = p.M <= kSkinnyMaxM ? 1 : split_factor(p.M, p.N, p.K);
    const size_t need = (size_t)s * p.M * p.N * 4;
    if (p.M <= kSkinnyMaxM) {
      launch_skinny<FA, FB>(p, stream);
    } else if (s > 1 && split_ws && used + need <= split_bytes) {
      orig[split.count] = &b.p[i];
      Problem &q = split.p[split.count++];
      q = p;
      q.c = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(split_ws) + used);
      q.splits = s;
      q.bias = nullptr;
      q.amax_out = nullptr;  // taken by the reduce kernel
      used += need;
    } else if (p.K < kMinBigK) {
      short_k.p[short_k.count++] = p;
    } else {
      rest.p[rest.count++] = p;
    }
  }
  if (split.count > 0) {
    int tiles = 0;
    for (int i = 0; i < split.count; ++i) {
      Problem &p = split.p[i];
      p.tiles_m = (p.M + 255) / 256;
      p.tiles_n = (p.N + 255) / 256;
      tiles += p.tiles_m * p.tiles_n * p.splits;
    }
    // short ranges take the eight-wave tiles (their per-tile prologue and
    // epilogue overlap between the two waves of a SIMD)
    int min_blocks = 1 << 30;
    for (int i = 0; i < split.count; ++i)
      min_blocks = std::min(min_blocks, ((split.p[i].K + kBK - 1) / kBK) / split.p[i].splits);
    if (min_blocks >= kSplitStagBlocks)
      gemm_fp8_tn_kernel<FA, FB, 256, 256, 2, 2, 1, 4, true><<<(unsigned)std::min(tiles, kCUs), 256, 0, stream>>>(split);
    else
      gemm_fp8_tn_kernel<FA, FB, 256, 256, 2, 4, 1, 4, true><<<(unsigned)std::min(tiles, kCUs), 512, 0, stream>>>(split);
  }
  // stag: 256 x 256 tiles take the four-wave kernel (at least four K
  // blocks), else the eight-wave one (2 x 4 waves of 128 x 64, two per SIMD,
  // the K loop of the smaller tiles)
  auto launch_rest = [&](Batch &rest, bool stag) {
    if (rest.count == 0) return;
    int64_t big = 0, small = 0;
    for (int i = 0; i < rest.count; ++i) {
      big += (int64_t)((rest.p[i].M + 255) / 256) * ((rest.p[i].N + 255) / 256);
      small += (int64_t)((rest.p[i].M + 127) / 128) * ((rest.p[i].N + 127) / 128);
    }
    // Problems whose tiles contract over different numbers of K blocks take
    // their tiles from a work queue, the longest problem first.
    bool mixed = false;
    for (int i = 1; i < rest.count; ++i)
      mixed |= (rest.p[i].K + kBK - 1) / kBK != (rest.p[0].K + kBK - 1) / kBK;
    // Big tiles, unless a ragged edge leaves their last round nearly empty:
    // the small tiles win when 0.75 x their rounds < the big rounds.  (With
    // the big tiles on 32 x 32 x 64 MFMAs the factor was 0.6: 12288 x 1600 x
    // 1600, 336 big tiles in two rounds 46.5 us, 1248 small ones in three
    // 43.0 us.  On 16 x 16 x 128 MFMAs the big tiles gained ~10% and now take
    // that shape too: the GPT-1.5B block's N = 1600 forwards, same box, step
    // 1367-1368 -> 1358-1360 us.)  A queued batch keeps the big tiles.
    const int64_t big_rounds = (big + kCUs - 1) / kCUs, small_rounds = (small + 2 * kCUs - 1) / (2 * kCUs);
    const bool use_big = big >= kCUs && ((mixed && queue) || 4 * big_rounds <= 3 * small_rounds);
    // At most one small tile per CU (e.g. 256 tokens: 64 tiles of 128 x 128):
    // tiles of 64 x 128 occupy twice as many CUs (measured: 1024 x 4096 x
    // 4096, 256 small tiles, 25.8 -> 24.1 us; from 384 small tiles on the
    // small ones are faster, 2048 x 4096 x 4096 34.9 vs 46.2 us).
    const bool use_med = !use_big && small <= kCUs;
    const int bm = use_big ? 256 : (use_med ? 64 : 128), bn = use_big ? 256 : 128;
    int tiles = 0;
    for (int i = 0; i < rest.count; ++i) {
      Problem &p = rest.p[i];
      p.tiles_m = (p.M + bm - 1) / bm;
      p.tiles_n = (p.N + bn - 1) / bn;
      p.splits = 1;
      tiles += p.tiles_m * p.tiles_n;
    }
    // With two or more waves of tiles per CU the output would only evict
    // operand lines from the caches: stream it (measured: -3.5% time at
    // 65536 x 4096 x 4096, +2% at 4096^3 where each CU writes one tile; from
    // two rounds instead of four, same box: 12288 x 4800 x 1600 101.8 ->
    // 99.9 us, 8192 x 4096 x 4096 102.0 -> 100.7 us, the 4096^3 backward
    // pair 102.9 -> 101.2 us).
    rest.nt_stores = tiles >= 2 * (use_big ? kCUs : 2 * kCUs);
    bool amax = false;
    for (int i = 0; i < rest.count; ++i) amax |= rest.p[i].amax_out != nullptr;
    // One problem whose last round of big tiles would be less than half full
    // (12288 x 1600: 336 tiles, a second round of 80): the tile rows of the
    // full rounds take the big tiles, the rows left over take one round of
    // small tiles in a launch of their own (measured, same box: 12288 x 1600
    // x 6400 119.8 -> 116.4 us, 12288 x 1600 x 1600 43.4 -> 42.9 us; two
    // small tiles on a CU run at about half a big tile's rate, so the gain
    // is small).
    if (use_big && rest.count == 1 && !mixed) {
      const Problem &p = rest.p[0];
      const int rounds = (tiles + kCUs - 1) / kCUs, last = tiles - (rounds - 1) * kCUs;
      const int rows_full = (rounds - 1) * kCUs / p.tiles_n * 256;
      const int small_left = ((p.M - rows_full + 127) / 128) * ((p.N + 127) / 128);
      if (rounds >= 2 && 2 * last < kCUs && rows_full > 0 && rows_full < p.M && small_left <= 2 * kCUs) {
        Batch head = rest, left = rest;
        head.p[0].M = rows_full;
        head.p[0].tiles_m = rows_full / 256;
        head.nt_stores = 0;
        const int head_tiles = head.p[0].tiles_m * head.p[0].tiles_n;
        if (stag)
          launch_tiled<FA, FB, 256, 256, 2, 2, 1, 4, false>(head, (unsigned)std::min(head_tiles, kCUs), amax, stream);
        else
          launch_tiled<FA, FB, 256, 256, 2, 4, 1, 4, false>(head, (unsigned)std::min(head_tiles, kCUs), amax, stream);
        Problem &q = left.p[0];
        q.M = p.M - rows_full;
        q.a = p.a + (int64_t)rows_full * p.lda;
        q.c = p.c + (int64_t)rows_full * p.N;
        left.nt_stores = 0;
        // (at most one 128 x 128 tile per CU: 64 x 128 tiles, as below)
        const bool med = small_left <= kCUs;
        q.tiles_m = (q.M + (med ? 63 : 127)) / (med ? 64 : 128);
        q.tiles_n = (q.N + 127) / 128;
        const int left_tiles = q.tiles_m * q.tiles_n;
        if (med)
          launch_tiled<FA, FB, 64, 128, 2, 2, 2, 8, false>(left, (unsigned)std::min(left_tiles, 2 * kCUs), amax, stream);
        else
          launch_tiled<FA, FB, 128, 128, 2, 2, 2, 8, false>(left, (unsigned)std::min(left_tiles, 2 * kCUs), amax,
                                                           stream);
        return;
      }
    }
    if (use_big && mixed && queue && fixed_stride_unbalanced(rest, std::min(tiles, kCUs))) {
      std::stable_sort(rest.p, rest.p + rest.count, [](const Problem &x, const Problem &y) { return x.K > y.K; });
      rest.queue = queue;
      if (stag)
        launch_tiled<FA, FB, 256, 256, 2, 2, 1, 4, true>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
      else
        launch_tiled<FA, FB, 256, 256, 2, 4, 1, 4, true>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
    } else if (use_big && tiles >= 8 * kCUs) {
      // Eight or more rounds of tiles: groups of eight tile-rows, so that an
      // XCD's 32 concurrent tiles form an 8 x 4 patch instead of 4 x 8
      // (measured, same box: 65536 x 4096 x 4096 forward 907 -> 878 us, its
      // backward pair 1682 -> 1669 us; with one to four rounds the two
      // patches are level within noise, or 4 x 8 is ahead: 4096^3 57.7 vs
      // 58.3 us).
      if (stag)
        launch_tiled<FA, FB, 256, 256, 2, 2, 1, 8, false>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
      else
        launch_tiled<FA, FB, 256, 256, 2, 4, 1, 8, false>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
    } else if (use_big) {
      if (stag)
        launch_tiled<FA, FB, 256, 256, 2, 2, 1, 4, false>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
      else
        launch_tiled<FA, FB, 256, 256, 2, 4, 1, 4, false>(rest, (unsigned)std::min(tiles, kCUs), amax, stream);
    } else if (use_med) {
      launch_tiled<FA, FB, 64, 128, 2, 2, 2, 8, false>(rest, (unsigned)std::min(tiles, 2 * kCUs), amax, stream);
    } else {
      launch_tiled<FA, FB, 128, 128, 2, 2, 2, 8, false>(rest, (unsigned)std::min(tiles, 2 * kCUs), amax, stream);
    }
  };
  launch_rest(rest, true);
  launch_rest(short_k, false);
  for (int i = 0; i < split.count; ++i) {
    const Problem &q = split.p[i];
    const int64_t mn = (int64_t)q.M * q.N;
    // with an amax, at most one workgroup per CU (one atomic each)
    const int64_t blocks = (mn / 4 + 255) / 256;
    const unsigned grid = (unsigned)(orig[i]->amax_out ? std::min<int64_t>(blocks, kCUs) : blocks);
    split_reduce_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<const float *>(q.c), q.splits, mn, q.inv_a,
                                                  q.inv_b, orig[i]->c, orig[i]->amax_out);
  }
}

}  // namespace

int split_factor(int64_t M, int64_t N, int64_t K) {
  // Few output tiles with a long contraction leave most CUs idle (e.g. a
  // weight gradient over many tokens with a small weight): split K into up
  // to eight ranges of at least eight 128-byte K blocks, so that the
  // (range, tile) pairs about fill the 256 CUs.
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (M <= kSkinnyMaxM || tiles == 0 || tiles * 2 > kCUs) return 1;
  const int64_t nkb = (K + kBK - 1) / kBK;
  int64_t s = std::min<int64_t>(kCUs / tiles, nkb / 8);
  s = std::min<int64_t>(s, 8);
  return s > 1 ? (int)s : 1;
}

size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = split_factor(M, N, K);
  return s > 1 ? (size_t)s * M * N * 4 : 0;
}

hipError_t launch_gemms(const GemmDesc *d, int count, int fmt_a, int fmt_b, hipStream_t stream, void *split_ws,
                        size_t split_bytes, uint32_t *queue) {
  Batch b{};
  for (int i = 0; i < count; ++i) {
    if (d[i].M == 0 || d[i].N == 0) continue;
    Problem &p = b.p[b.count++];
    p.a = d[i].a;
    p.b = d[i].b;
    p.inv_a = d[i].inv_a;
    p.inv_b = d[i].inv_b;
    p.c = d[i].c;
    p.bias = d[i].bias;
    p.amax_out = d[i].amax_out;
    p.M = (int)d[i].M;
    p.N = (int)d[i].N;
    p.K = (int)d[i].K;
    p.lda = (int)(d[i].lda ? d[i].lda : d[i].K);
    p.ldb = (int)(d[i].ldb ? d[i].ldb : d[i].K);
    p.splits = 1;
  }
  if (b.count == 0) return hipSuccess;
  float *ws = reinterpret_cast<float *>(split_ws);
  if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E4M3)
    launch_fmt<0, 0>(b, ws, split_bytes, queue, stream);
  else if (fmt_a == F8LIN_E5M2 && fmt_b == F8LIN_E4M3)
    launch_fmt<1, 0>(b, ws, split_bytes, queue, stream);
  else if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E5M2)
    launch_fmt<0, 1>(b, ws, split_bytes, queue, stream);
  else
    launch_fmt<1, 1>(b, ws, split_bytes, queue, stream);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N,
                       int64_t K, const float *inv_a, const float *inv_b, uint16_t *c, hipStream_t stream) {
  const GemmDesc d{a, b, inv_a, inv_b, c, M, N, K, nullptr};
  return launch_gemms(&d, 1, fmt_a, fmt_b, stream);
}

}  // namespace f8lin
