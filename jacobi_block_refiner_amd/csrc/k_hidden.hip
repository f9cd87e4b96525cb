// Pass-invariant hidden cache of an XPress step (gfx950).
//
// xh[n, b] = in_proj[:, 0:r] . (down_h . h[n, b]) + in_proj[:, r:2r] . (down_g . mean_b h[n, b])
// (vLLM API page "vllm.model_executor.models.qwen3_xpress", XPressRefinerHead.hidden_cache and the
// hidden half of in_proj that jacobi_refine_greedy applies once per step).
//
// The mean commutes with the linear map down_g, so down_g . mean_b h = mean_b (down_g . h[b]).
// That keeps both projections on exact bf16 operands: K1a runs one bf16 MFMA GEMM
// hdg = h . [down_h; down_g]^T over all N*B slot rows (fp32 accumulate), split over K into
// partial sums when there are few output tiles; K1b adds the partials in a fixed order, takes the
// slot mean of the down_g half and applies in_proj's hidden half in fp32.
#include "launch.hpp"
#include "xpress_common.hpp"

namespace xpress {

namespace {

constexpr int kTM = 64;  // rows (slots) per workgroup
constexpr int kTN = 64;  // output columns per workgroup
constexpr int kTK = 64;  // k chunk
constexpr int kLQ = kTK / 8 + 1;  // padded LDS row stride (uint4)

// Split-K partial products: part[ks, m, j] = sum_{k in slice ks} h[m, k] * Wcat[j, k].
// 4 waves as a 2 x 2 grid of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, layout as in the
// readout kernel: D[row = 8*(v/4) + 4*(l/32) + v%4][col = l%32]). The next k chunk is loaded into
// registers while the current one is multiplied out of LDS.
__global__ __launch_bounds__(256) void hidden_gemm_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ down_h,
                                                          const uint16_t* __restrict__ down_g,
                                                          int NB, int H, int r, int kslice,
                                                          float* __restrict__ part) {
  __shared__ uint4 s_a[kTM * kLQ];
  __shared__ uint4 s_b[kTN * kLQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
  const int ks = blockIdx.z;
  const int kbeg = ks * kslice, kend = min(H, kbeg + kslice);
  const int l32 = lane & 31, half = lane >> 5;
  // this thread's two 16-byte chunks of each k chunk: rows rr0, rr0 + 32 at column cc
  const int rr0 = tid / (kTK / 8), cc = tid % (kTK / 8);
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rr = rr0 + 32 * q;
    arow[q] = h + (int64_t)min(m0 + rr, NB - 1) * H;
    const int j = n0 + rr;  // output column = row of [down_h; down_g]
    brow[q] = (j < r) ? down_h + (int64_t)j * H : down_g + (int64_t)(j - r) * H;
  }
  uint4 ra[2], rb[2];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      ra[q] = reinterpret_cast<const uint4*>(arow[q] + k0)[cc];
      rb[q] = reinterpret_cast<const uint4*>(brow[q] + k0)[cc];
    }
  };
  f32x16 acc = {};
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kTK) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      s_a[(rr0 + 32 * q) * kLQ + cc] = ra[q];
      s_b[(rr0 + 32 * q) * kLQ + cc] = rb[q];
    }
    __syncthreads();
    if (k0 + kTK < kend) load(k0 + kTK);
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      const bf16x8 a = as_bf16x8(s_a[(32 * wm + l32) * kLQ + 2 * s + half]);
      const bf16x8 b = as_bf16x8(s_b[(32 * wn + l32) * kLQ + 2 * s + half]);
      acc = mfma32x32x16(a, b, acc);
    }
    __syncthreads();
  }
  const int col = n0 + 32 * wn + l32;
  float* out = part + (int64_t)ks * NB * (2 * r);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = m0 + 32 * wm + 8 * (v / 4) + 4 * half + (v % 4);
    if (row < NB) out[(int64_t)row * (2 * r) + col] = acc[v];
  }
}

// Split-K reduction, once per element, in a fixed order: hdg[m, j] = sum_s part[s, m, j].
__global__ __launch_bounds__(256) void hidden_reduce_kernel(const float4* __restrict__ part,
                                                            int nsplit, int64_t n4,
                                                            float4* __restrict__ hdg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  // splits in ascending order (fixed summation order); 8 loads in flight at a time
  float4 v = part[i];
  int sp = 1;
  for (; sp + 8 <= nsplit; sp += 8) {
    float4 u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = part[(sp + j) * n4 + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v.x += u[j].x;
      v.y += u[j].y;
      v.z += u[j].z;
      v.w += u[j].w;
    }
  }
  for (; sp < nsplit; ++sp) {
    const float4 u = part[sp * n4 + i];
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  hdg[i] = v;
}

// One workgroup per (block n, 64 output channels), in fp32:
//   hg[k] = (1/B) sum_b hdg[n, b, r + k]
//   xh[n, b, c] = sum_k P[c, k] hdg[n, b, k] + sum_k P[c, r + k] hg[k].
// hd and hg sit in LDS (read as broadcasts); each thread streams its in_proj row from L2.
template <int R>
__global__ __launch_bounds__(256) void hidden_project_kernel(const float* __restrict__ hdg,
                                                             const uint16_t* __restrict__ in_proj,
                                                             int B, float* __restrict__ xh) {
  __shared__ float s_hd[16][R];
  __shared__ float s_hg[R];
  __shared__ float s_gp[64];
  const int n = blockIdx.x, c0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int q = tid; q < 16 * R; q += 256) {
    const int b = q / R, k = q % R;
    s_hd[b][k] = b < B ? hdg[((int64_t)n * B + b) * 2 * R + k] : 0.f;
  }
  for (int k = tid; k < R; k += 256) {
    float sum = 0.f;
    for (int b = 0; b < B; ++b) sum += hdg[((int64_t)n * B + b) * 2 * R + R + k];
    s_hg[k] = sum / (float)B;
  }
  __syncthreads();
  const int c = tid & 63, grp = tid >> 6;  // grp: slots 4*grp .. 4*grp+3
  const uint4* prow = reinterpret_cast<const uint4*>(in_proj + (int64_t)(c0 + c) * 3 * R);
  if (grp == 0) {
    float g = 0.f;
    for (int kq = 0; kq < R / 8; ++kq) {
      const uint4 u = prow[R / 8 + kq];
      const float w8[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                           bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) g = fmaf(w8[e], s_hg[8 * kq + e], g);
    }
    s_gp[c] = g;
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kq = 0; kq < R / 8; ++kq) {
    const uint4 u = prow[kq];
    const float w8[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = fmaf(w8[e], s_hd[4 * grp + v][8 * kq + e], acc[v]);
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int b = 4 * grp + v;
    if (b < B) xh[((int64_t)n * B + b) * R + c0 + c] = acc[v] + s_gp[c];
  }
}

}  // namespace

// k chunks per split-K slice; every slice holds at least one chunk.
int hidden_chunks_per_split(int NB, int H, int r) {
  const int tiles = ((NB + kTM - 1) / kTM) * ((2 * r) / kTN);
  const int kchunks = H / kTK;
  int s = (512 + tiles - 1) / tiles;  // aim for >= 512 workgroups
  if (s > kchunks) s = kchunks;
  if (s < 1) s = 1;
  return (kchunks + s - 1) / s;
}

int hidden_splits(int NB, int H, int r) {
  const int cps = hidden_chunks_per_split(NB, H, r);
  return (H / kTK + cps - 1) / cps;
}

// split-K partials, then the reduced hdg [NB, 2r]
size_t hidden_scratch_bytes(int NB, int H, int r) {
  return ((size_t)hidden_splits(NB, H, r) + 1) * NB * 2 * r * sizeof(float);
}

// An upper bound of hidden_scratch_bytes over every H (the split count never exceeds the target
// number of splits, whatever H is).
size_t hidden_scratch_bytes_any_h(int NB, int r) {
  const int tiles = ((NB + kTM - 1) / kTM) * ((2 * r) / kTN);
  const int smax = (512 + tiles - 1) / tiles;
  return ((size_t)smax + 1) * NB * 2 * r * sizeof(float);
}

hipError_t launch_hidden_gemm(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                              int NB, int H, int r, float* part, hipStream_t s) {
  const int ns = hidden_splits(NB, H, r);
  const int kslice = hidden_chunks_per_split(NB, H, r) * kTK;
  dim3 grid((NB + kTM - 1) / kTM, (2 * r) / kTN, ns);
  hipLaunchKernelGGL(hidden_gemm_kernel, grid, dim3(256), 0, s, h, down_h, down_g, NB, H, r,
                     kslice, part);
  return hipGetLastError();
}

hipError_t launch_hidden_project(const float* part, int H, const uint16_t* in_proj, int N, int B,
                                 int r, float* xh, hipStream_t s) {
  const int NB = N * B;
  const int ns = hidden_splits(NB, H, r);
  float* hdg = const_cast<float*>(part) + (size_t)ns * NB * 2 * r;
  const int64_t n4 = (int64_t)NB * 2 * r / 4;
  hipLaunchKernelGGL(hidden_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(part), ns, n4, reinterpret_cast<float4*>(hdg));
  dim3 grid(N, r / 64);
  switch (r) {
    case 64:
      hipLaunchKernelGGL(hidden_project_kernel<64>, grid, dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    case 128:
      hipLaunchKernelGGL(hidden_project_kernel<128>, grid, dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    case 256:
      hipLaunchKernelGGL(hidden_project_kernel<256>, grid, dim3(256), 0, s, hdg, in_proj, B, xh);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace xpress
