// Per-step kernels of an XPress step (gfx950): the starting block and the pass bookkeeping of
// the device-side fixed-point exit.
#include "launch.hpp"
#include "block_start.hpp"
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

namespace {

// Starting block: one workgroup per draft row (the body is initial_block_row).
__global__ __launch_bounds__(256) void initial_block_kernel(const uint16_t* __restrict__ base,
                                                            int64_t ld,
                                                            const int64_t* __restrict__ anchor,
                                                            int B, int64_t V,
                                                            int64_t* __restrict__ blk) {
  initial_block_row(base, ld, anchor, B, V, blk, blockIdx.x);
}

// Serving form of the mixer (vLLM API page "vllm.model_executor.models.qwen3_xpress",
// XPressRefinerHead.fold_from_raw_): lower triangle kept, identity added, rounded to bf16.
__global__ void fold_mixer_kernel(const uint16_t* __restrict__ raw, int r, int B,
                                  uint16_t* __restrict__ mix_L) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)r * B * B;
  if (i >= n) return;
  const int j = (int)(i % B), b = (int)((i / B) % B), c = (int)(i / ((int64_t)B * B));
  float v = (j <= b) ? bf16_to_f32(raw[i]) : 0.f;
  if (j == b) v += 1.f;
  mix_L[((int64_t)b * B + j) * r + c] = f32_to_bf16(v);  // stored [B, B, r]
}

__global__ void set_anchor_kernel(const int64_t* anchor, int N, int B, int64_t* blk) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) blk[(int64_t)n * B] = anchor[n];
}

__global__ void flags_reset_kernel(int32_t* flags, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) flags[i] = 0;
}

// Pass p >= 1 ran iff pass p-1 changed a slot (flags[p-1] == 1); pass 0 always runs.
__global__ void count_passes_kernel(const int32_t* flags, int K, int stop, int32_t* passes_run) {
  if (threadIdx.x != 0) return;
  int n = K;
  if (stop && K > 0) {
    n = 1;
    for (int p = 0; p + 1 < K; ++p) n += flags[p] != 0;
  }
  *passes_run = n;
}

}  // namespace

hipError_t launch_initial_block(const uint16_t* base, int64_t ld, const int64_t* anchor, int N,
                                int B, int64_t V, int64_t* blk, hipStream_t s) {
  hipLaunchKernelGGL(initial_block_kernel, dim3(N * (B - 1)), dim3(256), 0, s, base, ld, anchor,
                     B, V, blk);
  return hipGetLastError();
}

hipError_t launch_fold_mixer(const uint16_t* raw, int r, int B, uint16_t* mix_L, hipStream_t s) {
  const int64_t n = (int64_t)r * B * B;
  hipLaunchKernelGGL(fold_mixer_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, raw, r,
                     B, mix_L);
  return hipGetLastError();
}

hipError_t launch_set_anchor(const int64_t* anchor, int N, int B, int64_t* blk, hipStream_t s) {
  hipLaunchKernelGGL(set_anchor_kernel, dim3((N + 255) / 256), dim3(256), 0, s, anchor, N, B, blk);
  return hipGetLastError();
}

hipError_t launch_flags_reset(int32_t* flags, int n, hipStream_t s) {
  hipLaunchKernelGGL(flags_reset_kernel, dim3(1), dim3(256), 0, s, flags, n);
  return hipGetLastError();
}

hipError_t launch_count_passes(const int32_t* flags, int K, int stop, int32_t* passes_run,
                               hipStream_t s) {
  hipLaunchKernelGGL(count_passes_kernel, dim3(1), dim3(64), 0, s, flags, K, stop, passes_run);
  return hipGetLastError();
}

}  // namespace xpress
