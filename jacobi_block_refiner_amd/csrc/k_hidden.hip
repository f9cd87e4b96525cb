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
// slot mean of the down_g half and applies in_proj's hidden half in fp32, one block of slots per
// workgroup.
#include "launch.hpp"
#include "block_start.hpp"
#include "hidden_tile.hpp"
#include "xpress_common.hpp"

namespace xpress {

namespace {

__global__ __launch_bounds__(256) void hidden_gemm_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ down_h,
                                                          const uint16_t* __restrict__ down_g,
                                                          int NB, int H, int r, int kslice,
                                                          float* __restrict__ part) {
  __shared__ GemmLds lds;
  hidden_gemm_tile<8>(h, down_h, down_g, NB, H, r, kslice, part, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// The start of a step in one launch: workgroups [0, g1) are the hidden GEMM's tiles (mt x nt
// tiles per split, split-major), the rest the starting block's rows. The two are independent; the
// GEMM is latency-bound and the starting block bandwidth-bound, so they overlap well. With
// zero_flags, workgroup 0 also clears the step's nzero pass flags (read only by later launches).
__global__ __launch_bounds__(256) void step_start_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ down_h,
    const uint16_t* __restrict__ down_g, int NB, int H, int r, int kslice,
    float* __restrict__ part, int g1, int mt, int nt, const uint16_t* __restrict__ base,
    int64_t ld, const int64_t* __restrict__ anchor, int B, int64_t V, int64_t* __restrict__ blk,
    int32_t* __restrict__ zero_flags, int nzero) {
  const int i = blockIdx.x;
  if (zero_flags && i == 0)
    for (int q = threadIdx.x; q < nzero; q += blockDim.x) zero_flags[q] = 0;
  __shared__ GemmLds lds;
  if (i < g1)
    hidden_gemm_tile<4>(h, down_h, down_g, NB, H, r, kslice, part, i % mt, (i / mt) % nt, i / (mt * nt), lds);
  else
    initial_block_row(base, ld, anchor, B, V, blk, i - g1);
}

// One workgroup per (block n, CW output channels), in fp32:
//   hdg[n, b, j] = sum_s part[s, n*B + b, j]            (splits in ascending order)
//   hg[k] = (1/B) sum_b hdg[n, b, r + k]                 (slots in ascending order)
//   xh[n, b, c] = sum_k P[c, k] hdg[n, b, k] + sum_k P[c, r + k] hg[k]
// The block's slots and its CW rows of in_proj's hidden half are staged in LDS with coalesced
// loads (many in flight); hd and hg are then read as broadcasts, the in_proj rows with a padded
// pitch (no bank conflicts). Thread (channel tid % CW, slot group tid / CW) computes CW/16
// slots. Fewer channels per workgroup give more workgroups (each re-reads the block's partials,
// L2 hits) and less arithmetic per thread; the launcher picks CW for about 256 workgroups.
template <int R, int CW>
__global__ __launch_bounds__(256) void hidden_project_kernel(const float* __restrict__ part,
                                                             int nsplit, int NB,
                                                             const uint16_t* __restrict__ in_proj,
                                                             int B, float* __restrict__ xh) {
  static_assert(CW == 16 || CW == 32 || CW == 64, "channels per workgroup");
  constexpr int PQ = 2 * R / 8;     // 16-byte chunks of a staged in_proj row
  constexpr int PP = PQ + 1;        // padded pitch
  constexpr int SPG = CW / 16;      // slots per thread
  __shared__ float s_hdg[16][2 * R];
  __shared__ float s_hg[R];
  __shared__ float s_gp[CW];
  __shared__ uint4 s_p[CW * PP];
  const int n = blockIdx.x, c0 = blockIdx.y * CW, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < CW * PQ / 256; ++i) {  // all of the thread's loads in flight together
    const int q = tid + 256 * i, row = q / PQ, col = q % PQ;
    s_p[row * PP + col] = reinterpret_cast<const uint4*>(in_proj + (int64_t)(c0 + row) * 3 * R)[col];
  }
  const int64_t n4 = (int64_t)NB * 2 * R / 4;  // float4s per split
  const float4* p4 = reinterpret_cast<const float4*>(part) + (int64_t)n * B * 2 * R / 4;
  const int nq = B * 2 * R / 4;
  auto add4 = [](float4& v, const float4& u) __attribute__((always_inline)) {
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  };
  // two float4s per thread at a time, splits in ascending order, eight splits per batch of loads
  for (int q0 = tid; q0 < nq; q0 += 512) {
    const int q1 = min(q0 + 256, nq - 1);  // a repeat of the last element when past the end
    float4 v0 = p4[q0], v1 = p4[q1];
    int sp = 1;
    for (; sp + 8 <= nsplit; sp += 8) {
      float4 u0[8], u1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u0[j] = p4[(sp + j) * n4 + q0];
        u1[j] = p4[(sp + j) * n4 + q1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        add4(v0, u0[j]);
        add4(v1, u1[j]);
      }
    }
    for (; sp < nsplit; ++sp) {
      add4(v0, p4[sp * n4 + q0]);
      add4(v1, p4[sp * n4 + q1]);
    }
    reinterpret_cast<float4*>(&s_hdg[0][0])[q0] = v0;
    if (q0 + 256 < nq) reinterpret_cast<float4*>(&s_hdg[0][0])[q0 + 256] = v1;
  }
  __syncthreads();
  for (int k = tid; k < R; k += 256) {
    float sum = 0.f;
    for (int b = 0; b < B; ++b) sum += s_hdg[b][R + k];
    s_hg[k] = sum / (float)B;
  }
  __syncthreads();
  const int c = tid % CW, grp = tid / CW;  // grp: slots SPG*grp .. SPG*grp+SPG-1
  const uint4* prow = s_p + c * PP;
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
  float acc[SPG];
#pragma unroll
  for (int v = 0; v < SPG; ++v) acc[v] = 0.f;
  const int b0 = SPG * grp;  // < 16
  for (int kq = 0; kq < R / 8; ++kq) {
    const uint4 u = prow[kq];
    const float w8[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                         bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int v = 0; v < SPG; ++v) acc[v] = fmaf(w8[e], s_hdg[b0 + v][8 * kq + e], acc[v]);
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < SPG; ++v) {
    const int b = SPG * grp + v;
    if (b < B) xh[((int64_t)n * B + b) * R + c0 + c] = acc[v] + s_gp[c];
  }
}

}  // namespace

// k chunks per split-K slice; every slice holds at least one chunk.
int hidden_chunks_per_split(int NB, int H, int r) {
  const int tiles = ((NB + kTM - 1) / kTM) * ((2 * r) / kTN);
  const int kchunks = H / kTK;
  // aim for >= 256 workgroups (one per CU), but at most kMaxSplits slices: every slice is one
  // more partial for the projection to read back (with few slot rows the GEMM is latency-bound
  // whatever the split)
  int s = (256 + tiles - 1) / tiles;
  if (s > kMaxSplits) s = kMaxSplits;
  // few slot rows: the projection's few workgroups each read every slice back, so fewer slices
  const int srow = max(2, (NB + kTM - 1) / kTM);
  if (s > srow) s = srow;
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
  const int smax = min((256 + tiles - 1) / tiles, kMaxSplits);
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

hipError_t launch_step_start(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                             int NB, int H, int r, float* part, const uint16_t* base, int64_t ld,
                             const int64_t* anchor, int N, int B, int64_t V, int64_t* blk,
                             hipStream_t s, int32_t* zero_flags, int nzero) {
  const int ns = hidden_splits(NB, H, r);
  const int kslice = hidden_chunks_per_split(NB, H, r) * kTK;
  const int mt = (NB + kTM - 1) / kTM, nt = (2 * r) / kTN;
  const int g1 = mt * nt * ns;
  hipLaunchKernelGGL(step_start_kernel, dim3((unsigned)(g1 + N * (B - 1))), dim3(256), 0, s, h,
                     down_h, down_g, NB, H, r, kslice, part, g1, mt, nt, base, ld, anchor, B, V,
                     blk, zero_flags, nzero);
  return hipGetLastError();
}

template <int R>
hipError_t launch_project_r(const float* part, int ns, int NB, const uint16_t* in_proj, int N,
                            int B, float* xh, hipStream_t s) {
  // the most channels per workgroup that still give >= 256 workgroups (16 below that)
  const int cw = N * (R / 64) >= 256 ? 64 : (N * (R / 32) >= 256 ? 32 : 16);
  switch (cw) {
    case 64:
      hipLaunchKernelGGL((hidden_project_kernel<R, 64>), dim3(N, R / 64), dim3(256), 0, s, part,
                         ns, NB, in_proj, B, xh);
      break;
    case 32:
      hipLaunchKernelGGL((hidden_project_kernel<R, 32>), dim3(N, R / 32), dim3(256), 0, s, part,
                         ns, NB, in_proj, B, xh);
      break;
    default:
      hipLaunchKernelGGL((hidden_project_kernel<R, 16>), dim3(N, R / 16), dim3(256), 0, s, part,
                         ns, NB, in_proj, B, xh);
  }
  return hipGetLastError();
}

hipError_t launch_hidden_project(const float* part, int H, const uint16_t* in_proj, int N, int B,
                                 int r, float* xh, hipStream_t s) {
  const int NB = N * B;
  const int ns = hidden_splits(NB, H, r);
  switch (r) {
    case 64: return launch_project_r<64>(part, ns, NB, in_proj, N, B, xh, s);
    case 128: return launch_project_r<128>(part, ns, NB, in_proj, N, B, xh, s);
    case 256: return launch_project_r<256>(part, ns, NB, in_proj, N, B, xh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xpress
