// Latent stage of one XPress pass (gfx950), as three wide kernels.
//
// For every block (vLLM API page "vllm.v1.worker.gpu.spec_decode.xpress.kernels",
// _xpress_latent_kernel docstring; "vllm.model_executor.models.qwen3_xpress",
// XPressRefinerHead._refine_latent):
//   1. gather the embedding of each slot's previous token: slot 0 reads am1, slot b reads blk[b-1];
//   2. x = xh + P_e . e with P_e = in_proj[:, 2r:3r];
//   3. per-channel causal mixer u[b, c] = sum_{j<=b} L[c, b, j] x[j, c];
//   4. SwiGLU: s = silu(w_gate . u) * (w_up . u);
//   5. lat = u + w_down . s for slots 1..B-1 (slot 0 is never read out).
// A block's 16 slots (padded with zero rows past B) are the M = 16 rows of a
// v_mfma_f32_16x16x32_bf16 tile. One workgroup per block cannot keep enough CUs busy at small N
// (each block-pass needs ~1 MB of weights, which one CU pulls from L2 in several microseconds), so
// the stage is split where a full reduction over channels is needed:
//   latent_mix_kernel   (block, 16-channel slice): steps 1-3, u in fp32 and bf16 to scratch;
//   latent_gate_kernel  (row tile, 64 hidden units): step 4, s in bf16 to scratch;
//   latent_down_kernel  (row tile, 64 channels): step 5, lat in bf16.
// Each workgroup reads at most 64 KB of weights; row tiles of 64 rows (4 blocks) share weight
// reads when there are many blocks.
//
// v_mfma_f32_16x16x32_bf16 operand layout (wave64):
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + e, e = 0..7
//   B (32 x 16): lane l holds col l%16, the same k
//   D (16 x 16): lane l, accumulator v holds row 4*(l/16) + v, col l%16
#include "launch.hpp"
#include "xpress_common.hpp"

namespace xpress {

namespace {

// Steps 1-3 for one block and 16 channels c0..c0+15; one wave.
template <int R>
__global__ __launch_bounds__(64) void latent_mix_kernel(
    const int64_t* __restrict__ blk, const int64_t* __restrict__ am1,
    const float* __restrict__ xh, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ in_proj, const uint16_t* __restrict__ mix_L, int B, int64_t V,
    float* __restrict__ u32, uint16_t* __restrict__ u16, const int32_t* __restrict__ flags,
    int pass) {
  if (pass_skipped(flags, pass)) return;
  __shared__ float s_x[16][17];
  const int n = blockIdx.x;
  const int c0 = blockIdx.y * 16;
  const int lane = threadIdx.x, l16 = lane & 15, q4 = lane >> 4;

  // token of slot l16 (slot 0 reads am1, slot b reads blk[b-1]); slots >= B and ids outside
  // [0, V) contribute a zero embedding
  int64_t tok = -1;
  if (l16 == 0) tok = am1[n];
  else if (l16 < B) tok = blk[(int64_t)n * B + l16 - 1];
  const bool live = tok >= 0 && tok < V;
  const uint4* erow = reinterpret_cast<const uint4*>(w1 + (live ? tok : 0) * R);
  const uint4* prow = reinterpret_cast<const uint4*>(in_proj + (int64_t)(c0 + l16) * 3 * R + 2 * R);

  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    uint4 e = erow[4 * s + q4];
    if (!live) e = make_uint4(0, 0, 0, 0);
    acc = mfma16x16x32(as_bf16x8(e), as_bf16x8(prow[4 * s + q4]), acc);
  }
  // x for slot 4*q4 + v, channel c0 + l16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int slot = 4 * q4 + v;
    const float h = slot < B ? xh[((int64_t)n * B + slot) * R + c0 + l16] : 0.f;
    s_x[slot][l16] = acc[v] + h;
  }
  __syncthreads();
  // mixer: this lane -> channel c0 + l16, slots 4*q4 .. 4*q4+3
  const int c = c0 + l16;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int b = 4 * q4 + v;
    float u = 0.f;
    if (b < B) {
      const uint16_t* lrow = mix_L + ((int64_t)c * B + b) * B;
      for (int j = 0; j <= b; ++j) u = fmaf(bf16_to_f32(lrow[j]), s_x[j][l16], u);
    }
    u32[((int64_t)n * 16 + b) * R + c] = u;
    u16[((int64_t)n * 16 + b) * R + c] = f32_to_bf16(u);
  }
}

// Step 4 for rows r0..r0+16*G-1 (whole blocks, 16 rows each) and hidden units h0..h0+63; wave w
// owns units h0 + 16w .. +15.
template <int R, int G>
__global__ __launch_bounds__(256) void latent_gate_kernel(
    const uint16_t* __restrict__ u16, const uint16_t* __restrict__ w_gate,
    const uint16_t* __restrict__ w_up, int M, int nrows, uint16_t* __restrict__ s16,
    const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int r0 = blockIdx.x * 16 * G;
  const int m = blockIdx.y * 64 + wave * 16 + l16;
  const uint4* grow = reinterpret_cast<const uint4*>(w_gate + (int64_t)m * R);
  const uint4* urow = reinterpret_cast<const uint4*>(w_up + (int64_t)m * R);
  f32x4 ag[G], au[G];
#pragma unroll
  for (int g = 0; g < G; ++g) ag[g] = au[g] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    const bf16x8 bg = as_bf16x8(grow[4 * s + q4]);
    const bf16x8 bu = as_bf16x8(urow[4 * s + q4]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int r = min(r0 + 16 * g + l16, nrows - 1);
      const bf16x8 a = as_bf16x8(reinterpret_cast<const uint4*>(u16 + (int64_t)r * R)[4 * s + q4]);
      ag[g] = mfma16x16x32(a, bg, ag[g]);
      au[g] = mfma16x16x32(a, bu, au[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * g + 4 * q4 + v;
      if (r < nrows) {
        const float x = ag[g][v];
        const float sg = x / (1.f + __expf(-x));
        s16[(int64_t)r * M + m] = f32_to_bf16(sg * au[g][v]);
      }
    }
}

// Step 5 for rows r0..r0+16*G-1 and channels c0..c0+63; wave w owns channels c0 + 16w .. +15.
template <int R, int G>
__global__ __launch_bounds__(256) void latent_down_kernel(
    const uint16_t* __restrict__ s16, const float* __restrict__ u32,
    const uint16_t* __restrict__ w_down, int M, int B, int nrows, uint16_t* __restrict__ lat,
    const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int r0 = blockIdx.x * 16 * G;
  const int c = blockIdx.y * 64 + wave * 16 + l16;
  const uint4* drow = reinterpret_cast<const uint4*>(w_down + (int64_t)c * M);
  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0, 0, 0, 0};
  for (int s = 0; s < M / 32; ++s) {
    const bf16x8 b = as_bf16x8(drow[4 * s + q4]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int r = min(r0 + 16 * g + l16, nrows - 1);
      const bf16x8 a = as_bf16x8(reinterpret_cast<const uint4*>(s16 + (int64_t)r * M)[4 * s + q4]);
      acc[g] = mfma16x16x32(a, b, acc[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * g + 4 * q4 + v;  // row = 16 * block + slot
      const int n = r >> 4, slot = r & 15;
      if (r < nrows && slot >= 1 && slot < B)
        lat[((int64_t)n * (B - 1) + slot - 1) * R + c] =
            f32_to_bf16(u32[(int64_t)r * R + c] + acc[g][v]);
    }
}

template <int R>
hipError_t launch_r(const int64_t* blk, const int64_t* am1, const float* xh, const uint16_t* w1,
                    const uint16_t* in_proj, const uint16_t* mix_L, const uint16_t* w_gate,
                    const uint16_t* w_up, const uint16_t* w_down, int N, int B, int M, int64_t V,
                    uint16_t* lat, void* scratch, const int32_t* flags, int pass, hipStream_t s) {
  const int nrows = N * 16;
  float* u32 = static_cast<float*>(scratch);
  uint16_t* u16 = reinterpret_cast<uint16_t*>(u32 + (size_t)nrows * R);
  uint16_t* s16 = u16 + (size_t)nrows * R;
  hipLaunchKernelGGL(latent_mix_kernel<R>, dim3(N, R / 16), dim3(64), 0, s, blk, am1, xh, w1,
                     in_proj, mix_L, B, V, u32, u16, flags, pass);
  const bool wide = N >= 128;  // 4 blocks per workgroup: weights read once per 64 rows
  const int G = wide ? 4 : 1;
  dim3 g2((nrows + 16 * G - 1) / (16 * G), M / 64), g3((nrows + 16 * G - 1) / (16 * G), R / 64);
  if (wide) {
    hipLaunchKernelGGL((latent_gate_kernel<R, 4>), g2, dim3(256), 0, s, u16, w_gate, w_up, M,
                       nrows, s16, flags, pass);
    hipLaunchKernelGGL((latent_down_kernel<R, 4>), g3, dim3(256), 0, s, s16, u32, w_down, M, B,
                       nrows, lat, flags, pass);
  } else {
    hipLaunchKernelGGL((latent_gate_kernel<R, 1>), g2, dim3(256), 0, s, u16, w_gate, w_up, M,
                       nrows, s16, flags, pass);
    hipLaunchKernelGGL((latent_down_kernel<R, 1>), g3, dim3(256), 0, s, s16, u32, w_down, M, B,
                       nrows, lat, flags, pass);
  }
  return hipGetLastError();
}

}  // namespace

size_t latent_scratch_bytes(int N, int r, int M) {
  const size_t nrows = (size_t)N * 16;
  return nrows * r * 4 + nrows * r * 2 + nrows * M * 2;
}

hipError_t launch_latent(const int64_t* blk, const int64_t* am1, const float* xh,
                         const uint16_t* w1, const uint16_t* in_proj, const uint16_t* mix_L,
                         const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                         int N, int B, int r, int M, int64_t V, uint16_t* lat, void* scratch,
                         const int32_t* flags, int pass, hipStream_t s) {
  switch (r) {
    case 64: return launch_r<64>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s);
    case 128: return launch_r<128>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s);
    case 256: return launch_r<256>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xpress
