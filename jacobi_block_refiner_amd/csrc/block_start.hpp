// Starting block of a step (shared by the standalone kernel and the fused step-start kernel).
#pragma once
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

// Starting block (vLLM API page "vllm.model_executor.models.qwen3_xpress",
// jacobi_refine_greedy), draft row p by one workgroup of 256 threads: blk[n, b] =
// argmax_v base[p, v] with the lowest id on ties; the first row of each block also stores the
// anchor in slot 0.
__device__ __forceinline__ void initial_block_row(const uint16_t* __restrict__ base, int64_t ld,
                                                  const int64_t* __restrict__ anchor, int B,
                                                  int64_t V, int64_t* __restrict__ blk, int p) {
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int tid = threadIdx.x;
  const uint16_t* row = base + (int64_t)p * ld;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const int64_t nq = V / 8;
  const uint4* rq = reinterpret_cast<const uint4*>(row);
  auto scan = [&](const uint4& u, int id) __attribute__((always_inline)) {
    const float v8[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool gt = v8[e] > bv;
      bv = gt ? v8[e] : bv;
      bi = gt ? id + e : bi;
    }
  };
  // four independent 16-byte loads in flight per thread; a thread's ids only increase, so the
  // strict > keeps its lowest id among equal values
  int64_t q = tid;
  for (; q + 3 * 256 < nq; q += 4 * 256) {
    const uint4 u0 = rq[q], u1 = rq[q + 256], u2 = rq[q + 512], u3 = rq[q + 768];
    scan(u0, (int)(q * 8));
    scan(u1, (int)((q + 256) * 8));
    scan(u2, (int)((q + 512) * 8));
    scan(u3, (int)((q + 768) * 8));
  }
  for (; q < nq; q += 256) scan(rq[q], (int)(q * 8));
  for (int64_t v = nq * 8 + tid; v < V; v += 256) argmax_merge(bv, bi, bf16_to_f32(row[v]), (int)v);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    argmax_merge(bv, bi, ov, oi);
  }
  if ((tid & 63) == 0) {
    s_v[tid >> 6] = bv;
    s_i[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, s_v[w], s_i[w]);
    // nothing rose above -inf (a row of -inf, or NaN): the lowest id, 0, as for equal values
    if (bi == INT_MAX) bi = 0;
    const int n = p / (B - 1), b = 1 + p % (B - 1);
    blk[(int64_t)n * B + b] = bi;
    if (b == 1) blk[(int64_t)n * B] = anchor[n];
  }
}

}  // namespace xpress
