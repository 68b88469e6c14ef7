// fp8 GEMM with a per-tensor dequantisation epilogue, for all three GEMMs of
// the Float8Linear forward + backward (pytorch/torchtitan PR #778,
// "Benchmarking single linear layer forward+backward performance"):
//   C (M, N) bf16 = (A (M, K) . B (N, K)^T) * inv_a * inv_b
// Both operands are K-contiguous ("TN"); the cast kernel writes the
// transposed fp8 copies so that forward, dgrad and wgrad all take this form.
//
// gfx950 design (each choice measured on MI355X):
//   * v_mfma_f32_32x32x64_f8f6f4 (the scaled builtin with zero scale operands
//     selects the unscaled instruction); e4m3 / e5m2 per operand through
//     cbsz / blgp.  A lane feeds the same 32 K-bytes of its A row and of its
//     B row, so A and B share one K order and the instruction's internal K
//     order cannot matter.
//   * Two waves per SIMD: one wave per SIMD reached only ~75-85% of the MFMA
//     rate in an issue-rate probe, two waves ~97%.  Workgroups:
//       big   256 x 256 tile, 8 waves (2 x 4), wave tile 128 x 64
//             (128 fp32 accumulators per lane), one workgroup per CU;
//       small 128 x 128 tile, 4 waves (2 x 2), wave tile 64 x 64, two per CU,
//             for shapes with too few big tiles to fill 256 CUs.
//   * K step of 128 bytes, two LDS stages.  Global -> LDS copies use
//     buffer_load_dwordx4 ... lds (no register staging); eight lanes fetch
//     one 128-byte row line.  The buffer resource's range check returns
//     zeros for rows past M / N, and K chunks past K are pointed outside the
//     range, so ragged edges load zeros with no branches.
//   * LDS slot of (row r, 16-byte chunk c) = r*8 + (c ^ ((r>>1) & 7)): every
//     16 consecutive rows at one chunk fall in 16 distinct bank groups, so
//     the 128-bit fragment reads are conflict-free.
//   * Fragments are refilled in place right after their last use, so the
//     next sub-step's LDS reads overlap the current MFMAs with one register
//     set; one barrier per K step, placed after the first row of MFMAs of the
//     second sub-step, both publishes stage k+1 and retires stage k.
//   * Epilogue: fp32 accumulator * (inv_a * inv_b) rounded once to bf16
//     (nearest even), staged through LDS per wave and written as 16-byte
//     row segments.
#include "device_common.h"
#include "internal.h"

namespace f8lin {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 128;
// Every matrix dimension is at most 2^22 (checked at the C ABI), so a tile's
// byte range rows * K stays below 2^31 and this offset is always outside it.
constexpr int kOutOfRange = (int)0x80000000u;

__device__ __forceinline__ int slot128(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their no-wait maxima
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Tile of workgroup b.  Workgroups are dispatched round-robin over the 8
// XCDs (b -> XCD b % 8), and each XCD has its own L2, so XCD x is given the
// contiguous tile range [x*T/8, (x+1)*T/8), walked in groups of G tile-rows,
// column by column: the tiles an XCD runs at once form a compact patch
// (G tile-rows x a few tile-columns) whose A and B slices its L2 shares.
// With row-major order an XCD's concurrent tiles spanned many tile-rows and
// each XCD re-fetched them (measured: 4.5x the operand bytes past L2).
template <int G>
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int T = tiles_m * tiles_n;
  const int per = T / 8;
  int t = b;
  if (b < per * 8) t = (b % 8) * per + b / 8;
  const int gsize = G * tiles_n;
  const int grp = t / gsize, in = t % gsize;
  const int gm = min(G, tiles_m - grp * G);
  tm = grp * G + in % gm;
  tn = in / gm;
}

template <int FA, int FB, int BM, int BN, int WAVES_M, int WAVES_N, int MIN_BLOCKS, int G>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MIN_BLOCKS) void gemm_fp8_tn_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ inv_a, const float *__restrict__ inv_b, uint16_t *__restrict__ C, int tiles_m,
    int tiles_n) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;            // 32x32 MFMA tiles per wave
  constexpr int OPA = BM * kBK, OPB = BN * kBK;          // bytes per operand per stage
  constexpr int STB = OPA + OPB;
  constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW);  // 1 KB copies per wave per stage
  static_assert(LA >= 1 && LB >= 1 && TM >= 2 && TN >= 1, "tile configuration");
  static_assert(NW * WTM * WTN * 2 <= 2 * STB, "epilogue staging must fit in LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tm, tn;
  tile_of<G>((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void *)(A + (int64_t)m0 * K), (short)0, rows_a * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void *)(B + (int64_t)n0 * K), (short)0, rows_b * K, 0x00020000);

  // Global offset (without the K step base) and K byte of each 16-byte slot
  // this lane copies: slot s = (wave * L + j) * 64 + lane.
  int offa[LA], kca[LA], offb[LB], kcb[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int s = (wave * LA + j) * 64 + lane;
    const int r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
    offa[j] = r * K + c * 16;
    kca[j] = c * 16;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int s = (wave * LB + j) * 64 + lane;
    const int r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
    offb[j] = r * K + c * 16;
    kcb[j] = c * 16;
  }
  auto issue = [&](int kt) {
    const int k0 = kt * kBK;
    uint8_t *stage = smem + (kt & 1) * STB;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int vo = (kca[j] + k0 < K) ? offa[j] + k0 : kOutOfRange;  // past K: outside the range -> 0
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void *)(stage + (wave * LA + j) * 1024), 16, vo, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int vo = (kcb[j] + k0 < K) ? offb[j] + k0 : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void *)(stage + OPA + (wave * LB + j) * 1024), 16, vo, 0,
                                               0, 0);
    }
  };

  const int wm = (wave / WAVES_N) * WTM, wn = (wave % WAVES_N) * WTN;
  const int g = lane >> 5;  // K half within a 64-byte sub-step
  int arow[TM], brow[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = wm + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < TN; ++j) brow[j] = wn + j * 32 + (lane & 31);

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Fragment of row r for sub-step ks (0/1) of the K step in `stage`:
  // chunks ks*4 + g*2 and +1 (32 K-bytes).
  auto rd = [&](int stage, int op_off, int r, int ks) {
    const u32x4 *st = (const u32x4 *)(smem + stage * STB + op_off);
    const int c = ks * 4 + g * 2;
    const u32x4 lo = st[slot128(r, c)], hi = st[slot128(r, c + 1)];
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto mfma = [&](const v8i &a, const v8i &b, v16f &c) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
  };

  v8i fa[TM], fb[TN];
  const int nk = (K + kBK - 1) / kBK;
  if (nk > 0) {
    issue(0);
    wait_vmcnt0();
    __builtin_amdgcn_s_barrier();
    if (nk > 1) issue(1);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = rd(0, 0, arow[i], 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = rd(0, OPA, brow[j], 0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    // sub-step 0: fragments hold (kt, 0); refill with (kt, 1)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        mfma(fa[i], fb[j], acc[i][j]);
        if (i == TM - 1) fb[j] = rd(cur, OPA, brow[j], 1);
      }
      fa[i] = rd(cur, 0, arow[i], 1);
    }
    // sub-step 1: after its first row, stage kt+1 is resident (every wave waited
    // for its own copies, then the barrier) and every wave is done with stage
    // kt, whose buffer then receives stage kt+2.
#pragma unroll
    for (int j = 0; j < TN; ++j) mfma(fa[0], fb[j], acc[0][j]);
    if (more) {
      wait_vmcnt0();
      __builtin_amdgcn_s_barrier();
      if (kt + 2 < nk) issue(kt + 2);
      fa[0] = rd(cur ^ 1, 0, arow[0], 0);
    }
#pragma unroll
    for (int i = 1; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        mfma(fa[i], fb[j], acc[i][j]);
        if (i == TM - 1 && more) fb[j] = rd(cur ^ 1, OPA, brow[j], 0);
      }
      if (more) fa[i] = rd(cur ^ 1, 0, arow[i], 0);
    }
  }

  // Epilogue: each wave stages its WTM x WTN bf16 tile in its own LDS region
  // (rows of WTN*2 bytes, 64-byte halves swapped on rows with bit 2 set to
  // spread the two row groups of a store over different banks), then writes
  // 16-byte row segments.
  __syncthreads();
  constexpr int RB = WTN * 2;
  const float alpha = inv_a[0] * inv_b[0];
  uint8_t *wreg = smem + wave * (WTM * RB);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = j * 32 + (lane & 31);
        *(uint16_t *)(wreg + row * RB + ((col * 2) ^ (((row >> 2) & 1) << 6))) =
            (uint16_t)f32_to_bf16_rne(acc[i][j][v] * alpha);
      }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < WTM * CPR / 64; ++it) {
    const int idx = it * 64 + lane;
    const int row = idx / CPR, ch = idx % CPR;
    const u32x4 v = *(const u32x4 *)(wreg + row * RB + ((ch * 16) ^ (((row >> 2) & 1) << 6)));
    const int grow = m0 + wm + row, gcol = n0 + wn + ch * 8;
    if (grow < M && gcol < N) *(u32x4 *)(C + (int64_t)grow * N + gcol) = v;
  }
}

template <int FA, int FB>
void launch_fmt(const uint8_t *a, const uint8_t *b, int M, int N, int K, const float *ia, const float *ib,
                uint16_t *c, hipStream_t stream) {
  constexpr int kCUs = 256;
  const int64_t big = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (big >= kCUs) {
    const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
    gemm_fp8_tn_kernel<FA, FB, 256, 256, 2, 4, 1, 4>
        <<<(unsigned)big, 512, 0, stream>>>(a, b, M, N, K, ia, ib, c, tiles_m, tiles_n);
  } else {
    const int tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
    const int64_t small = (int64_t)tiles_m * tiles_n;
    gemm_fp8_tn_kernel<FA, FB, 128, 128, 2, 2, 2, 8>
        <<<(unsigned)small, 256, 0, stream>>>(a, b, M, N, K, ia, ib, c, tiles_m, tiles_n);
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N,
                       int64_t K, const float *inv_a, const float *inv_b, uint16_t *c, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E4M3)
    launch_fmt<0, 0>(a, b, m, n, k, inv_a, inv_b, c, stream);
  else if (fmt_a == F8LIN_E5M2 && fmt_b == F8LIN_E4M3)
    launch_fmt<1, 0>(a, b, m, n, k, inv_a, inv_b, c, stream);
  else if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E5M2)
    launch_fmt<0, 1>(a, b, m, n, k, inv_a, inv_b, c, stream);
  else
    launch_fmt<1, 1>(a, b, m, n, k, inv_a, inv_b, c, stream);
  return hipGetLastError();
}

}  // namespace f8lin
