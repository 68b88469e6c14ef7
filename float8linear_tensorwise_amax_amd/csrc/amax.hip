// Tensorwise amax of a bf16 tensor, two algorithms (the ATOMIC_MAX and
// REDUCTION kernel_algo rows of the single-linear-layer table in
// pytorch/torchtitan PR #778):
//   atomic : one launch; each workgroup reduces its grid-stride share and folds
//            it with an atomic max into the slot of its group (workgroup
//            index mod 8); the last workgroup of a group (ticket counter)
//            folds the group into the tensor's slot the same way, and the
//            last group to do so publishes the result.  Every slot and
//            ticket is cleared again for the next call.
//   twopass: the same per-workgroup reduction writes one partial per
//            workgroup; the second pass reduces them -- inside the prologue of
//            the cast kernel that consumes the amax (f8lin_forward /
//            f8lin_backward), or as a one-workgroup launch (f8lin_amax).
// Both compute max |x| exactly as the max of the 15-bit magnitude fields, so
// both give the same bits as a plain max over |x| in any order.  One launch
// may reduce two tensors (the forward's X and W) with separate workgroups,
// slots and partials per tensor.
//
// HBM-bound: 2 bytes read per element.  Loads are 128-bit (8 bf16), sixteen
// in flight per thread per iteration.  The grid is at most one 512-thread
// workgroup per CU (256) per tensor, striding over the tensor: on MI355X
// device-wide atomics on one address are serialised beyond the per-XCD L2s
// (about 10 ns each, measured), so the atomic variant keeps the number of
// workgroups small and spreads their atomics over eight group slots, one
// 128-byte line each (eight-way less serialisation per address).  Fewer,
// fuller waves start sooner than many short ones (measured: 512 threads x 16
// loads beat 1024 x 8 by 4-6% on 64-512 MiB tensors).  Loads are ordinary
// (cached): the cast that follows re-reads the same tensor and can hit in the
// last-level cache when the tensor fits.
#include "device_common.h"
#include "internal.h"

namespace f8lin {
namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 16;
static_assert(kMaxGrid * kMaxAmaxTensors + kWsPartialsOffset <= (int)(kWorkspaceBytes / 4),
              "partials do not fit the workspace");

// Max magnitude (15-bit) over this thread's grid-stride share of x[0, n).
// The grid sweeps the tensor from its end to its start: the cast that
// follows walks it from the start, so the last lines this pass leaves in the
// last-level cache are the first ones the cast reads (measured, same box: the
// 65536-row linear's amax + cast of X and W 311 -> 306 us, of dY 292 -> 287
// us, its step 3067 -> 3050 us).
__device__ __forceinline__ uint32_t thread_magmax(const uint16_t *__restrict__ x, int64_t n, int64_t gtid,
                                                  int64_t nthreads) {
  const u32x4 *__restrict__ xv = reinterpret_cast<const u32x4 *>(x);
  const int64_t nv = n >> 3;  // whole 8-element vectors
  uint32_t m = 0;
  int64_t i = gtid;
  for (; i + (kUnroll - 1) * nthreads < nv; i += kUnroll * nthreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = xv[nv - 1 - (i + u * nthreads)];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      m = mag_max2(m, v[u].x);
      m = mag_max2(m, v[u].y);
      m = mag_max2(m, v[u].z);
      m = mag_max2(m, v[u].w);
    }
  }
  for (; i < nv; i += nthreads) {
    const u32x4 v = xv[nv - 1 - i];
    m = mag_max2(m, v.x);
    m = mag_max2(m, v.y);
    m = mag_max2(m, v.z);
    m = mag_max2(m, v.w);
  }
  const int64_t tail = n - (nv << 3);  // < 8 trailing elements
  if (gtid < tail) m = max(m, (uint32_t)x[(nv << 3) + gtid] & 0x7FFFu);
  return m;
}

// Workgroup max; the result is valid in thread 0.
__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v = max(v, red[w]);
    v = max(v, red[0]);
  }
  return v;
}

// One launch can reduce up to kMaxAmaxTensors tensors: workgroups
// [first[t], first[t] + grid[t]) belong to tensor t.
struct AmaxJob {
  const uint16_t *x;
  int64_t n;
  float *out;
  int first;
  int grid;
};
struct AmaxJobs {
  AmaxJob j[kMaxAmaxTensors];
  int count;
};

__device__ __forceinline__ int job_of(const AmaxJobs &jobs) {
  int t = 0;
#pragma unroll
  for (int i = 1; i < kMaxAmaxTensors; ++i)
    if (i < jobs.count && (int)blockIdx.x >= jobs.j[i].first) t = i;
  return t;
}

// Folds m into slot [0] (running max) and takes a ticket from slot [1]; true
// for the last of `members` callers, which gets the slot's final max in
// `all` and leaves the slot cleared.
//
// No fence: device-scope atomics are performed at one coherence point, and a
// fence here (an L2 write-back plus invalidate of the whole XCD cache on this
// chip) cost more than the reduction itself.  The order that matters -- each
// caller's max performed before its ticket -- comes from a data dependency
// instead: the ticket's operand uses the value the max returned, so it cannot
// issue before the max has completed.  Slot values are 15-bit magnitudes, so
// prev >> 15 is always 0 and the ticket adds exactly 1.  The last caller
// reads and clears the max with one exchange, issued only after its ticket
// came back, so every member's max is in.
__device__ __forceinline__ bool fold_last(uint32_t *slot, uint32_t m, uint32_t members, uint32_t &all) {
  const uint32_t prev = atomicMax(&slot[0], m);
  if (atomicAdd(&slot[1], 1u + (prev >> 15)) != members - 1) return false;
  all = atomicExch(&slot[0], 0u);
  atomicExch(&slot[1], 0u);
  return true;
}

__global__ __launch_bounds__(kThreads) void amax_atomic_kernel(const AmaxJobs jobs, uint32_t *ws) {
  const int t = job_of(jobs);
  const AmaxJob &jb = jobs.j[t];
  const int64_t nthreads = (int64_t)jb.grid * kThreads;
  const int lb = (int)blockIdx.x - jb.first;
  const int64_t gtid = (int64_t)lb * kThreads + threadIdx.x;
  const uint32_t m = block_max(thread_magmax(jb.x, jb.n, gtid, nthreads));
  if (threadIdx.x == 0) {
    const int grp = lb % kAmaxGroups;
    const uint32_t members = (uint32_t)((jb.grid - grp + kAmaxGroups - 1) / kAmaxGroups);
    const uint32_t groups = (uint32_t)min(jb.grid, kAmaxGroups);
    uint32_t gm, all;
    if (fold_last(ws + kWsGroupOffset + kWsSlotWords * (kAmaxGroups * t + grp), m, members, gm) &&
        fold_last(ws + kWsSlotWords * t, gm, groups, all))
      jb.out[0] = __uint_as_float(all << 16);
  }
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const AmaxJobs jobs, uint32_t *__restrict__ ws) {
  const int t = job_of(jobs);
  const AmaxJob &jb = jobs.j[t];
  const int64_t nthreads = (int64_t)jb.grid * kThreads;
  const int64_t lb = blockIdx.x - jb.first;
  const int64_t gtid = lb * kThreads + threadIdx.x;
  const uint32_t m = block_max(thread_magmax(jb.x, jb.n, gtid, nthreads));
  if (threadIdx.x == 0) ws[kWsPartialsOffset + t * kMaxGrid + lb] = m;
}

// One workgroup per tensor reduces that tensor's partials and clears them,
// so the workspace is zero again.
__global__ __launch_bounds__(kThreads) void amax_final_kernel(const AmaxJobs jobs, uint32_t *__restrict__ ws) {
  const int t = blockIdx.x;
  uint32_t *partials = ws + kWsPartialsOffset + t * kMaxGrid;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < jobs.j[t].grid; i += kThreads) {
    m = max(m, partials[i]);
    partials[i] = 0u;
  }
  m = block_max(m);
  if (threadIdx.x == 0) jobs.j[t].out[0] = __uint_as_float(m << 16);
}

int grid_for(int64_t n) {
  const int64_t nv = n >> 3;
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  int64_t g = (nv + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > kMaxGrid) g = kMaxGrid;
  return (int)g;
}

}  // namespace

hipError_t launch_amax(const AmaxTensor *ts, int count, int algo, uint32_t *ws, hipStream_t stream) {
  AmaxJobs jobs = {};
  jobs.count = count;
  int total = 0;
  for (int t = 0; t < count; ++t) {
    jobs.j[t] = AmaxJob{ts[t].x, ts[t].n, ts[t].out, total, grid_for(ts[t].n)};
    total += jobs.j[t].grid;
  }
  if (algo == F8LIN_AMAX_ATOMIC) {
    amax_atomic_kernel<<<total, kThreads, 0, stream>>>(jobs, ws);
  } else {
    amax_partial_kernel<<<total, kThreads, 0, stream>>>(jobs, ws);
    amax_final_kernel<<<count, kThreads, 0, stream>>>(jobs, ws);
  }
  return hipGetLastError();
}

hipError_t launch_amax_partials(const AmaxTensor *ts, int count, uint32_t *ws, const uint32_t **parts, int *nparts,
                                hipStream_t stream) {
  AmaxJobs jobs = {};
  jobs.count = count;
  int total = 0;
  for (int t = 0; t < count; ++t) {
    jobs.j[t] = AmaxJob{ts[t].x, ts[t].n, ts[t].out, total, grid_for(ts[t].n)};
    parts[t] = ws + kWsPartialsOffset + t * kMaxGrid;
    nparts[t] = jobs.j[t].grid;
    total += jobs.j[t].grid;
  }
  amax_partial_kernel<<<total, kThreads, 0, stream>>>(jobs, ws);
  return hipGetLastError();
}

}  // namespace f8lin
