// Ceiling probes for MI355X (gfx950): what this chip sustains on the two
// resources the Float8Linear path is bound by, measured with kernels of the
// same shape as the path's own, so that the path's kernels can be read
// against them.  Measurement tooling (libf8lin_probe.so, driven by
// `bench.py --ceilings`); nothing on the path calls it.
//
//   f8probe_stream: HBM streaming with 128-bit accesses, grid-stride over a
//     buffer, in three forms -- read only (a max over the words, one result
//     per workgroup), write only (a constant), and copy (read + write) -- the
//     access patterns of the amax pass (read), and of the cast (read 2 B,
//     write 2 B per element).
//   f8probe_mfma: v_mfma_f32_32x32x64_f8f6f4 back to back from registers,
//     eight independent accumulator tiles per wave (the 128 x 64 wave tile of
//     the GEMM), two waves per SIMD, one workgroup of eight waves per CU; each
//     workgroup records s_memtime (shader clock) and s_memrealtime (a
//     constant 100 MHz) around its loop, so the host derives the clock the
//     matrix cores ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kUnroll = 8;

// mode 0: read (max of words -> out[block]); 1: write (constant); 2: copy.
template <int MODE>
__global__ __launch_bounds__(512) void stream_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                      int64_t nvec, uint32_t *__restrict__ out) {
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t m = 0;
  for (; i + (kUnroll - 1) * nthreads < nvec; i += kUnroll * nthreads) {
    if constexpr (MODE == 1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[i + u * nthreads] = u32x4{(uint32_t)i, 1u, 2u, 3u};
    } else {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * nthreads];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if constexpr (MODE == 0) {
          m = max(m, max(max(v[u].x, v[u].y), max(v[u].z, v[u].w)));
        } else {
          dst[i + u * nthreads] = v[u];
        }
      }
    }
  }
  for (; i < nvec; i += nthreads) {
    if constexpr (MODE == 0) {
      const u32x4 v = src[i];
      m = max(m, max(max(v.x, v.y), max(v.z, v.w)));
    } else if constexpr (MODE == 1) {
      dst[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
    } else {
      dst[i] = src[i];
    }
  }
  if constexpr (MODE == 0) {
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(out + blockIdx.x, m);
  }
}

// Eight accumulator tiles per wave, `iters` rounds of eight MFMAs.  The
// operands are built from the thread index so the compiler cannot fold them;
// the accumulators' sum is stored once, so the loop cannot be removed.  The
// 128 accumulators and 48 operand registers (~178 VGPRs) allow two waves per
// SIMD, so each CU holds one workgroup of eight waves, as the GEMM does.
__global__ __launch_bounds__(512) void mfma_kernel(int iters, float *__restrict__ sink, uint64_t *__restrict__ clocks) {
  v8i a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = v8i{(int)threadIdx.x + i, 1, 2, 3, 4, 5, 6, 7};
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = v8i{(int)threadIdx.x ^ j, 7, 6, 5, 4, 3, 2, 1};
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// mode: 0 read, 1 write, 2 copy; n_bytes a multiple of 16; out: one word per
// workgroup (read mode; zeroed by the caller).  Returns a hipError_t.
int f8probe_stream(int mode, const void *src, void *dst, int64_t n_bytes, int grid, int block, uint32_t *out,
                   void *stream) {
  if (mode < 0 || mode > 2 || n_bytes < 0 || n_bytes % 16 || grid < 1 || block < 64 || block > 512 || block % 64)
    return (int)hipErrorInvalidValue;
  if ((mode != 1 && !src) || (mode != 0 && !dst) || (mode == 0 && !out)) return (int)hipErrorInvalidValue;
  const int64_t nvec = n_bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  const u32x4 *sp = (const u32x4 *)src;
  u32x4 *dp = (u32x4 *)dst;
  if (mode == 0)
    stream_kernel<0><<<grid, block, 0, s>>>(sp, dp, nvec, out);
  else if (mode == 1)
    stream_kernel<1><<<grid, block, 0, s>>>(sp, dp, nvec, out);
  else
    stream_kernel<2><<<grid, block, 0, s>>>(sp, dp, nvec, out);
  return (int)hipGetLastError();
}

// grid workgroups of 512 threads (eight waves); sink: grid * 512 floats;
// clocks: 2 * grid uint64 {shader-clock cycles, 100 MHz ticks} per workgroup.
// Flops: grid * 8 waves * iters * 8 * 131072.
int f8probe_mfma(int grid, int iters, float *sink, uint64_t *clocks, void *stream) {
  if (grid < 1 || iters < 1 || !sink || !clocks) return (int)hipErrorInvalidValue;
  mfma_kernel<<<grid, 512, 0, (hipStream_t)stream>>>(iters, sink, clocks);
  return (int)hipGetLastError();
}

}  // extern "C"
