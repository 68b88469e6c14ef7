// Host-side launchers of the gfx950 kernels (one per kernel family), called by
// the C-ABI layer in api.hip after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/f8lin.h"

namespace f8lin {

// Workspace layout (uint32 words): [0] atomic-max accumulator, [1] ticket,
// [64, 64 + kAmaxMaxBlocks) two-pass partial maxima.
constexpr int kAmaxMaxBlocks = 1024;
constexpr int kWsPartialsOffset = 64;
constexpr size_t kWorkspaceBytes = 8192;
static_assert((kWsPartialsOffset + kAmaxMaxBlocks) * 4 <= kWorkspaceBytes, "workspace too small");

hipError_t launch_amax(const uint16_t *x, int64_t n, int algo, float *amax_out, uint32_t *ws,
                       hipStream_t stream);

hipError_t launch_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, int fmt, int mode,
                                 const f8lin_state &st, uint8_t *q, uint8_t *qt, hipStream_t stream);

hipError_t launch_cast_f32(const float *v, int64_t n, int fmt, uint8_t *q, hipStream_t stream);

hipError_t launch_gemm(const uint8_t *a, int fmt_a, const uint8_t *b, int fmt_b, int64_t M, int64_t N,
                       int64_t K, const float *inv_a, const float *inv_b, uint16_t *c, hipStream_t stream);

hipError_t launch_delayed_update(const f8lin_state *states, int n, hipStream_t stream);

}  // namespace f8lin
