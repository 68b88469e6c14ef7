// fp8 GEMM with a per-tensor dequantisation epilogue, for all three GEMMs of
// the Float8Linear forward + backward (pytorch/torchtitan PR #778,
// "Benchmarking single linear layer forward+backward performance"):
//   C (M, N) bf16 = (A (M, K) . B (N, K)^T) * inv_a * inv_b
// Both operands are K-contiguous ("TN"); the cast kernel writes the
// transposed fp8 copies so that forward, dgrad and wgrad all take this form.
//
// gfx950 design:
//   * v_mfma_f32_32x32x64_f8f6f4 (the scaled builtin with zero scale operands,
//     which selects the unscaled instruction); operand formats per GEMM
//     (e4m3 x e4m3 forward, e5m2 x e4m3 backward) through cbsz / blgp.
//     Each lane feeds 32 consecutive K bytes of one row of A and the same 32
//     K bytes of one row of B, so A and B share one K ordering and the
//     hardware's internal K order inside an instruction cannot matter.
//   * 256 threads (4 waves in 2 x 2), 128 x 128 output tile, each wave
//     64 x 64 (2 x 2 MFMA tiles, 64 fp32 accumulators per lane).
//   * K step 128 bytes: global -> registers (128-bit loads) for step k+1
//     while step k's MFMAs read the other LDS buffer; one barrier per step.
//   * LDS rows of 128 bytes with 16-byte chunks XOR-swizzled by row % 8, so
//     both the 128-bit stores and the 128-bit fragment reads are conflict-free.
//   * Edges: rows beyond M / N and K chunks beyond K load as zero (every
//     dimension is a multiple of 16 and chunks are 16 bytes); stores are masked.
//   * Epilogue: fp32 accumulator * (inv_a * inv_b), rounded once to bf16
//     (nearest even).
#include "device_common.h"
#include "internal.h"

namespace f8lin {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <int FA, int FB>
__global__ __launch_bounds__(kThreads, 2) void gemm_fp8_tn_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, int M, int N, int K,
    const float *__restrict__ inv_a, const float *__restrict__ inv_b, uint16_t *__restrict__ C, int tiles_n) {
  __shared__ u32x4 sA[2][kBM * 8];
  __shared__ u32x4 sB[2][kBN * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m0 = (int)(blockIdx.x / tiles_n) * kBM;
  const int n0 = (int)(blockIdx.x % tiles_n) * kBN;
  const int lrow = tid >> 3;   // loader row (plus 32 * i)
  const int lchunk = tid & 7;  // loader 16-byte chunk within the K step

  const u32x4 zero = {0, 0, 0, 0};
  u32x4 ra[4], rb[4];
  auto load = [&](int kt) {
    const int gk = kt * kBK + lchunk * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 32 * i;
      const int gm = m0 + r;
      const int gn = n0 + r;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4 *>(A + (int64_t)gm * K + gk) : zero;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4 *>(B + (int64_t)gn * K + gk) : zero;
    }
  };
  auto store = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lrow + 32 * i;
      sA[st][swz(r, lchunk)] = ra[i];
      sB[st][swz(r, lchunk)] = rb[i];
    }
  };

  const int wm = (wave >> 1) * 64;
  const int wn = (wave & 1) * 64;
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + kBK - 1) / kBK;
  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c0 = ks * 4 + (lane >> 5) * 2;  // two 16-byte chunks = 32 K bytes
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm + i * 32 + (lane & 31);
        const u32x4 lo = sA[cur][swz(r, c0)];
        const u32x4 hi = sA[cur][swz(r, c0 + 1)];
        fa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn + j * 32 + (lane & 31);
        const u32x4 lo = sB[cur][swz(r, c0)];
        const u32x4 hi = sB[cur][swz(r, c0 + 1)];
        fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], FA, FB, 0, 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane l, register v holds
  // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
  const float alpha = inv_a[0] * inv_b[0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M && col < N) C[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v] * alpha);
      }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N,
                       int64_t K, const float *inv_a, const float *inv_b, uint16_t *c, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  const unsigned grid = (unsigned)tiles_m * (unsigned)tiles_n;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E4M3)
    gemm_fp8_tn_kernel<0, 0><<<grid, kThreads, 0, stream>>>(a, b, m, n, k, inv_a, inv_b, c, tiles_n);
  else if (fmt_a == F8LIN_E5M2 && fmt_b == F8LIN_E4M3)
    gemm_fp8_tn_kernel<1, 0><<<grid, kThreads, 0, stream>>>(a, b, m, n, k, inv_a, inv_b, c, tiles_n);
  else if (fmt_a == F8LIN_E4M3 && fmt_b == F8LIN_E5M2)
    gemm_fp8_tn_kernel<0, 1><<<grid, kThreads, 0, stream>>>(a, b, m, n, k, inv_a, inv_b, c, tiles_n);
  else
    gemm_fp8_tn_kernel<1, 1><<<grid, kThreads, 0, stream>>>(a, b, m, n, k, inv_a, inv_b, c, tiles_n);
  return hipGetLastError();
}

}  // namespace f8lin
