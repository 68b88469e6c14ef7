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
//     matrix cores ran at.  The operands are either small constants built
//     from the thread index or random codes loaded once from a buffer: the
//     matrix cores draw more power when their inputs toggle, and the clock
//     shows it.
//   f8probe_mfma_shape: the 256 x 256 tile's MFMA stream from registers, one
//     wave per SIMD (four per workgroup), 128 x 128 outputs per wave, random
//     codes: as 16 accumulator blocks of v_mfma_f32_32x32x64_f8f6f4 or as 64
//     of v_mfma_f32_16x16x128_f8f6f4 -- the two instructions draw different
//     power per flop, so the clock the chip holds differs.
//   f8probe_mfma_lds: the GEMM's K loop without its global -> LDS copies: the
//     same waves and MFMAs, each wave reading its A and B fragments for every
//     64-byte K step from two 64 KB LDS stages (256 A rows and 256 B rows of
//     128 bytes, 16-byte chunks XOR-swizzled by row pair, the GEMM's layout),
//     filled once with random codes; the next step's fragments are read while
//     the current step's MFMAs run, and the workgroup meets at a barrier once
//     per 128-byte K block, as the GEMM does.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

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
// operands are built from the thread index (ops == nullptr) or loaded from
// ops (48 words per thread, thread-major), so the compiler cannot fold them;
// the accumulators' sum is stored once, so the loop cannot be removed.  The
// 128 accumulators and 48 operand registers (~178 VGPRs) allow two waves per
// SIMD, so each CU holds one workgroup of eight waves, as the GEMM does.
__global__ __launch_bounds__(512) void mfma_kernel(int iters, const int *__restrict__ ops, float *__restrict__ sink,
                                                   uint64_t *__restrict__ clocks) {
  v8i a[4], b[2];
  if (ops) {
    const int *p = ops + (int64_t)(blockIdx.x * blockDim.x + threadIdx.x) * 48;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[i][e] = p[i * 8 + e];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) b[j][e] = p[32 + j * 8 + e];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = v8i{(int)threadIdx.x + i, 1, 2, 3, 4, 5, 6, 7};
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = v8i{(int)threadIdx.x ^ j, 7, 6, 5, 4, 3, 2, 1};
  }
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

// One wave per SIMD, 128 x 128 outputs per wave: SHAPE 0 = 4 x 4 blocks of
// 32 x 32 x 64, SHAPE 1 = 8 x 8 blocks of 16 x 16 x 128; operands are 128
// int32 words per thread from ops (thread-major), loaded once.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_shape_kernel(int iters, const int *__restrict__ ops, float *__restrict__ sink,
                                                         uint64_t *__restrict__ clocks) {
  constexpr int NF = SHAPE == 0 ? 4 : 8;  // fragments per operand
  v8i a[NF], b[NF];
  const int *p = ops + (int64_t)(blockIdx.x * blockDim.x + threadIdx.x) * 128;
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = p[i * 8 + e];
      b[i][e] = p[64 + i * 8 + e];
    }
  typedef typename std::conditional<SHAPE == 0, v16f, v4f>::type acc_t;
  acc_t acc[NF][NF];
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = acc_t{};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        if constexpr (SHAPE == 0)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
      }
  }
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < (SHAPE == 0 ? 16 : 4); ++v) sum += acc[i][j][v];
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// 16-byte chunk c (0..7) of LDS row r (0..511) of one 64 KB stage.
__device__ __forceinline__ int chunk_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Fragment of row r for 64-byte K step ks (0/1) of a stage: lanes 0-31 take
// the step's first 32 bytes, lanes 32-63 the second 32.
__device__ __forceinline__ v8i lds_frag(const u32x4 *st, int r, int ks) {
  const int c = ks * 4 + (threadIdx.x & 32 ? 2 : 0);
  const u32x4 lo = st[chunk_slot(r, c)], hi = st[chunk_slot(r, c + 1)];
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// `iters` K blocks of 128 bytes over two LDS stages filled once from src
// (8192 chunks of 16 bytes); per block and wave: 16 MFMAs, 24 fragment reads
// of 16 bytes, one barrier.
__global__ __launch_bounds__(512) void mfma_lds_kernel(const u32x4 *__restrict__ src, int iters,
                                                       float *__restrict__ sink, uint64_t *__restrict__ clocks) {
  __shared__ __attribute__((aligned(1024))) u32x4 st[2 * 4096];
  for (int i = threadIdx.x; i < 2 * 4096; i += blockDim.x) st[i] = src[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave / 4) * 128, wn = 256 + (wave % 4) * 64;  // B rows follow the 256 A rows
  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  v8i fa[4], fb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = lds_frag(st, wm + i * 32 + (lane & 31), 0);
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[j] = lds_frag(st, wn + j * 32 + (lane & 31), 0);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // the next step: this block's second half, or the next block's first
      const u32x4 *nst = st + ((ks == 0 ? it : it + 1) & 1) * 4096;
      const int nks = ks ^ 1;
      v8i na[4], nb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) na[i] = lds_frag(nst, wm + i * 32 + (lane & 31), nks);
#pragma unroll
      for (int j = 0; j < 2; ++j) nb[j] = lds_frag(nst, wn + j * 32 + (lane & 31), nks);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = na[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = nb[j];
    }
    __syncthreads();
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

// grid workgroups of 512 threads (eight waves); ops: NULL (operands from the
// thread index) or grid * 512 * 48 int32 words of operand codes; sink:
// grid * 512 floats; clocks: 2 * grid uint64 {shader-clock cycles, 100 MHz
// ticks} per workgroup.  Flops: grid * 8 waves * iters * 8 * 131072.
int f8probe_mfma(int grid, int iters, const void *ops, float *sink, uint64_t *clocks, void *stream) {
  if (grid < 1 || iters < 1 || !sink || !clocks) return (int)hipErrorInvalidValue;
  mfma_kernel<<<grid, 512, 0, (hipStream_t)stream>>>(iters, (const int *)ops, sink, clocks);
  return (int)hipGetLastError();
}

// shape 0 (32 x 32 x 64) or 1 (16 x 16 x 128); grid workgroups of 256 threads;
// ops: grid * 256 * 128 int32 words of operand codes; sink: grid * 256 floats;
// clocks as above.  Flops: grid * 4 waves * iters * 2 * 128 * 128 * (64 for
// shape 0, 128 for shape 1).
int f8probe_mfma_shape(int shape, int grid, int iters, const void *ops, float *sink, uint64_t *clocks, void *stream) {
  if (shape < 0 || shape > 1 || grid < 1 || iters < 1 || !ops || !sink || !clocks) return (int)hipErrorInvalidValue;
  if (shape == 0)
    mfma_shape_kernel<0><<<grid, 256, 0, (hipStream_t)stream>>>(iters, (const int *)ops, sink, clocks);
  else
    mfma_shape_kernel<1><<<grid, 256, 0, (hipStream_t)stream>>>(iters, (const int *)ops, sink, clocks);
  return (int)hipGetLastError();
}

// As f8probe_mfma, fragments read from LDS: src holds 131072 bytes of
// operand codes (two 64 KB stages) that every workgroup copies in once.
// Flops: grid * 8 waves * iters * 16 * 131072.
int f8probe_mfma_lds(int grid, int iters, const void *src, float *sink, uint64_t *clocks, void *stream) {
  if (grid < 1 || iters < 1 || !src || !sink || !clocks) return (int)hipErrorInvalidValue;
  mfma_lds_kernel<<<grid, 512, 0, (hipStream_t)stream>>>((const u32x4 *)src, iters, sink, clocks);
  return (int)hipGetLastError();
}

}  // extern "C"
