// Pass-invariant hidden cache of an XPress step (gfx950).
//
// xh[n, b] = in_proj[:, 0:r] . (down_h . h[n, b]) + in_proj[:, r:2r] . (down_g . mean_b h[n, b])
// (vLLM API page "vllm.model_executor.models.qwen3_xpress", XPressRefinerHead.hidden_cache and the
// hidden half of in_proj that jacobi_refine_greedy applies once per step).
//
// The mean commutes with the linear map down_g, so down_g . mean_b h = mean_b (down_g . h[b]).
// That keeps both projections on exact bf16 operands: K1a runs one bf16 MFMA GEMM
// hdg = h . [down_h; down_g]^T over all N*B slot rows (fp32 accumulate, fp32 out), and K1b takes
// the slot mean of the down_g half and applies in_proj's hidden half in fp32.
#include "launch.hpp"
#include "xpress_common.hpp"

namespace xpress {

namespace {

constexpr int kTM = 64;  // rows (slots) per workgroup
constexpr int kTN = 64;  // output columns per workgroup
constexpr int kTK = 64;  // k chunk
constexpr int kLQ = kTK / 8 + 1;  // padded LDS row stride (uint4)

// 4 waves as a 2 x 2 grid of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, layout as in the
// readout kernel: D[row = 8*(v/4) + 4*(l/32) + v%4][col = l%32]).
__global__ __launch_bounds__(256) void hidden_gemm_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ down_h,
                                                          const uint16_t* __restrict__ down_g,
                                                          int NB, int H, int r,
                                                          float* __restrict__ hdg) {
  __shared__ uint4 s_a[kTM * kLQ];
  __shared__ uint4 s_b[kTN * kLQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
  const int l32 = lane & 31, half = lane >> 5;
  f32x16 acc = {};
  for (int k0 = 0; k0 < H; k0 += kTK) {
    for (int q = tid; q < kTM * (kTK / 8); q += 256) {
      const int rr = q / (kTK / 8), cc = q % (kTK / 8);
      uint4 va = make_uint4(0, 0, 0, 0);
      if (m0 + rr < NB) va = reinterpret_cast<const uint4*>(h + (int64_t)(m0 + rr) * H + k0)[cc];
      s_a[rr * kLQ + cc] = va;
      const int j = n0 + rr;  // output column = row of [down_h; down_g]
      const uint16_t* wrow = (j < r) ? down_h + (int64_t)j * H : down_g + (int64_t)(j - r) * H;
      s_b[rr * kLQ + cc] = reinterpret_cast<const uint4*>(wrow + k0)[cc];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      const bf16x8 a = as_bf16x8(s_a[(32 * wm + l32) * kLQ + 2 * s + half]);
      const bf16x8 b = as_bf16x8(s_b[(32 * wn + l32) * kLQ + 2 * s + half]);
      acc = mfma32x32x16(a, b, acc);
    }
    __syncthreads();
  }
  const int col = n0 + 32 * wn + l32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + 32 * wm + 8 * (v / 4) + 4 * half + (v % 4);
    if (row < NB) hdg[(int64_t)row * (2 * r) + col] = acc[v];
  }
}

// One workgroup per block n: mean of the down_g half over the B slots, then in_proj's hidden half.
template <int R>
__global__ __launch_bounds__(256) void hidden_project_kernel(const float* __restrict__ hdg,
                                                             const uint16_t* __restrict__ in_proj,
                                                             int B, float* __restrict__ xh) {
  __shared__ float s_hd[16][R];
  __shared__ float s_hg[R];
  const int n = blockIdx.x, tid = threadIdx.x;
  const float* base = hdg + (int64_t)n * B * (2 * R);
  for (int q = tid; q < B * R; q += 256) s_hd[q / R][q % R] = base[(int64_t)(q / R) * 2 * R + q % R];
  for (int k = tid; k < R; k += 256) {
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += base[(int64_t)b * 2 * R + R + k];
    s_hg[k] = s / (float)B;
  }
  __syncthreads();
  for (int i = tid; i < R; i += 256) {
    float acc[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[b] = 0.f;
    float g = 0.f;
    const uint4* prow = reinterpret_cast<const uint4*>(in_proj + (int64_t)i * 3 * R);
    for (int kq = 0; kq < R / 8; ++kq) {
      const uint4 p1 = prow[kq];
      const uint4 p2 = prow[R / 8 + kq];
      const float w1v[8] = {bf16_lo(p1.x), bf16_hi(p1.x), bf16_lo(p1.y), bf16_hi(p1.y),
                            bf16_lo(p1.z), bf16_hi(p1.z), bf16_lo(p1.w), bf16_hi(p1.w)};
      const float w2v[8] = {bf16_lo(p2.x), bf16_hi(p2.x), bf16_lo(p2.y), bf16_hi(p2.y),
                            bf16_lo(p2.z), bf16_hi(p2.z), bf16_lo(p2.w), bf16_hi(p2.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kq * 8 + e;
        g = fmaf(w2v[e], s_hg[k], g);
#pragma unroll
        for (int b = 0; b < 16; ++b)
          if (b < B) acc[b] = fmaf(w1v[e], s_hd[b][k], acc[b]);
      }
    }
    for (int b = 0; b < B; ++b) xh[((int64_t)n * B + b) * R + i] = acc[b] + g;
  }
}

}  // namespace

hipError_t launch_hidden_gemm(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                              int NB, int H, int r, float* hdg, hipStream_t s) {
  dim3 grid((NB + kTM - 1) / kTM, (2 * r) / kTN);
  hipLaunchKernelGGL(hidden_gemm_kernel, grid, dim3(256), 0, s, h, down_h, down_g, NB, H, r, hdg);
  return hipGetLastError();
}

hipError_t launch_hidden_project(const float* hdg, const uint16_t* in_proj, int N, int B, int r,
                                 float* xh, hipStream_t s) {
  switch (r) {
    case 64:
      hipLaunchKernelGGL(hidden_project_kernel<64>, dim3(N), dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    case 128:
      hipLaunchKernelGGL(hidden_project_kernel<128>, dim3(N), dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    case 256:
      hipLaunchKernelGGL(hidden_project_kernel<256>, dim3(N), dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace xpress
