// Fused latent stage of one XPress pass (gfx950).
//
// One workgroup (4 waves) computes one block end to end (vLLM API page
// "vllm.v1.worker.gpu.spec_decode.xpress.kernels", _xpress_latent_kernel docstring; "vllm.
// model_executor.models.qwen3_xpress", XPressRefinerHead._refine_latent):
//   1. gather the embedding of each slot's previous token: slot 0 reads am1, slot b reads
//      blk[b-1];
//   2. x = xh + P_e . e with P_e = in_proj[:, 2r:3r]  (16-slot x r MFMA GEMM, fp32 accumulate);
//   3. per-channel causal mixer u[b, c] = sum_{j<=b} L[c, b, j] x[j, c] in fp32;
//   4. SwiGLU: s = silu(w_gate . u) * (w_up . u)  (MFMA, silu in fp32);
//   5. lat = u + w_down . s for slots 1..B-1 (slot 0 is never read out), stored as bf16.
// The 16 slots of a block are exactly the M = 16 rows of a v_mfma_f32_16x16x32_bf16 tile (slots
// beyond B are zero padding). Activations live in LDS; weights stream from L2 straight into the
// MFMA B operands (each weight row is K-contiguous in the nn.Linear layout).
#include "launch.hpp"
#include "xpress_common.hpp"

namespace xpress {

namespace {

// v_mfma_f32_16x16x32_bf16 operand layout (wave64):
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + e, e = 0..7
//   B (32 x 16): lane l holds col l%16, the same k
//   D (16 x 16): lane l, accumulator v holds row 4*(l/16) + v, col l%16
template <int R, int M>
__global__ __launch_bounds__(256) void latent_kernel(
    const int64_t* __restrict__ blk, const int64_t* __restrict__ am1,
    const float* __restrict__ xh, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ in_proj, const uint16_t* __restrict__ mix_L,
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ w_down, int B, int64_t V, uint16_t* __restrict__ lat,
    const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int RQ = R / 8;   // uint4 per r-row
  constexpr int MQ = M / 8;   // uint4 per M-row
  constexpr int ELD = RQ + 1; // padded LDS strides (uint4)
  constexpr int SLD = MQ + 1;
  constexpr int XLD = R + 4;  // fp32 row stride
  constexpr int NT_R = R / 64;  // 16-wide channel tiles per wave
  constexpr int NT_M = M / 64;  // 16-wide hidden tiles per wave

  __shared__ int64_t s_tok[16];
  __shared__ uint4 s_e[16 * ELD];    // gathered embeddings, then u in bf16
  __shared__ float s_x[16 * XLD];    // x
  __shared__ float s_u[16 * XLD];    // u (fp32, residual)
  __shared__ uint4 s_s[16 * SLD];    // SwiGLU output in bf16

  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;

  if (tid < 16) {
    int64_t t = -1;
    if (tid == 0) t = am1[n];
    else if (tid < B) t = blk[(int64_t)n * B + tid - 1];
    s_tok[tid] = t;
  }
  __syncthreads();
  for (int q = tid; q < 16 * RQ; q += 256) {
    const int slot = q / RQ, cc = q % RQ;
    const int64_t t = s_tok[slot];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t >= 0 && t < V) v = reinterpret_cast<const uint4*>(w1 + t * R)[cc];  // ids outside [0, V) read as zero
    s_e[slot * ELD + cc] = v;
  }
  __syncthreads();

  // 2. x = xh + e . P_e^T ; wave w owns channels [w*R/4, (w+1)*R/4)
  {
    const int c0 = wave * (R / 4);
    f32x4 acc[NT_R];
#pragma unroll
    for (int t = 0; t < NT_R; ++t) acc[t] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < R / 32; ++s) {
      const bf16x8 a = as_bf16x8(s_e[l16 * ELD + 4 * s + q4]);
#pragma unroll
      for (int t = 0; t < NT_R; ++t) {
        const int ch = c0 + 16 * t + l16;
        const uint4 bq = reinterpret_cast<const uint4*>(in_proj + (int64_t)ch * 3 * R + 2 * R)[4 * s + q4];
        acc[t] = mfma16x16x32(a, as_bf16x8(bq), acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT_R; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int slot = 4 * q4 + v, ch = c0 + 16 * t + l16;
        const float h = (slot < B) ? xh[((int64_t)n * B + slot) * R + ch] : 0.f;
        s_x[slot * XLD + ch] = acc[t][v] + h;
      }
  }
  __syncthreads();

  // 3. causal mixer: thread -> (slot b = tid % 16, channels tid/16 + 16 k)
  {
    const int b = tid & 15;
    uint16_t* s_ub = reinterpret_cast<uint16_t*>(s_e);
    for (int c = tid >> 4; c < R; c += 16) {
      float u = 0.f;
      if (b < B) {
        const uint16_t* lrow = mix_L + ((int64_t)c * B + b) * B;
        for (int j = 0; j <= b; ++j) u = fmaf(bf16_to_f32(lrow[j]), s_x[j * XLD + c], u);
      }
      s_u[b * XLD + c] = u;
      s_ub[b * (ELD * 8) + c] = f32_to_bf16(u);
    }
  }
  __syncthreads();

  // 4. SwiGLU hidden: wave w owns hidden units [w*M/4, (w+1)*M/4)
  {
    const int h0 = wave * (M / 4);
    f32x4 ag[NT_M], au[NT_M];
#pragma unroll
    for (int t = 0; t < NT_M; ++t) ag[t] = au[t] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < R / 32; ++s) {
      const bf16x8 a = as_bf16x8(s_e[l16 * ELD + 4 * s + q4]);
#pragma unroll
      for (int t = 0; t < NT_M; ++t) {
        const int m = h0 + 16 * t + l16;
        const uint4 gq = reinterpret_cast<const uint4*>(w_gate + (int64_t)m * R)[4 * s + q4];
        const uint4 uq = reinterpret_cast<const uint4*>(w_up + (int64_t)m * R)[4 * s + q4];
        ag[t] = mfma16x16x32(a, as_bf16x8(gq), ag[t]);
        au[t] = mfma16x16x32(a, as_bf16x8(uq), au[t]);
      }
    }
    uint16_t* s_sb = reinterpret_cast<uint16_t*>(s_s);
#pragma unroll
    for (int t = 0; t < NT_M; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int slot = 4 * q4 + v, m = h0 + 16 * t + l16;
        const float g = ag[t][v];
        const float sg = g / (1.f + __expf(-g));
        s_sb[slot * (SLD * 8) + m] = f32_to_bf16(sg * au[t][v]);
      }
  }
  __syncthreads();

  // 5. lat = u + s . w_down^T ; wave w owns channels [w*R/4, (w+1)*R/4)
  {
    const int c0 = wave * (R / 4);
    f32x4 acc[NT_R];
#pragma unroll
    for (int t = 0; t < NT_R; ++t) acc[t] = f32x4{0, 0, 0, 0};
#pragma unroll 4
    for (int s = 0; s < M / 32; ++s) {
      const bf16x8 a = as_bf16x8(s_s[l16 * SLD + 4 * s + q4]);
#pragma unroll
      for (int t = 0; t < NT_R; ++t) {
        const int ch = c0 + 16 * t + l16;
        const uint4 dq = reinterpret_cast<const uint4*>(w_down + (int64_t)ch * M)[4 * s + q4];
        acc[t] = mfma16x16x32(a, as_bf16x8(dq), acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < NT_R; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int slot = 4 * q4 + v, ch = c0 + 16 * t + l16;
        if (slot >= 1 && slot < B)
          lat[((int64_t)n * (B - 1) + slot - 1) * R + ch] =
              f32_to_bf16(s_u[slot * XLD + ch] + acc[t][v]);
      }
  }
}

template <int R>
hipError_t launch_r(const int64_t* blk, const int64_t* am1, const float* xh, const uint16_t* w1,
                    const uint16_t* in_proj, const uint16_t* mix_L, const uint16_t* w_gate,
                    const uint16_t* w_up, const uint16_t* w_down, int N, int B, int M, int64_t V,
                    uint16_t* lat, const int32_t* flags, int pass, hipStream_t s) {
#define XP_LAT(MM)                                                                           \
  case MM:                                                                                   \
    hipLaunchKernelGGL((latent_kernel<R, MM>), dim3(N), dim3(256), 0, s, blk, am1, xh, w1,   \
                       in_proj, mix_L, w_gate, w_up, w_down, B, V, lat, flags, pass);        \
    break;
  switch (M) {
    XP_LAT(64)
    XP_LAT(128)
    XP_LAT(256)
    XP_LAT(512)
    XP_LAT(1024)
    default: return hipErrorInvalidValue;
  }
#undef XP_LAT
  return hipGetLastError();
}

}  // namespace

hipError_t launch_latent(const int64_t* blk, const int64_t* am1, const float* xh,
                         const uint16_t* w1, const uint16_t* in_proj, const uint16_t* mix_L,
                         const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                         int N, int B, int r, int M, int64_t V, uint16_t* lat,
                         const int32_t* flags, int pass, hipStream_t s) {
  switch (r) {
    case 64: return launch_r<64>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, flags, pass, s);
    case 128: return launch_r<128>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, flags, pass, s);
    case 256: return launch_r<256>(blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, flags, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xpress
