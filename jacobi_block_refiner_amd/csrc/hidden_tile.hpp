// Split-K bf16 MFMA tile of the hidden cache's GEMM (shared by the kernels that run it beside
// other independent work in one launch).
#pragma once

#include "xpress_common.hpp"

namespace xpress {

namespace {

constexpr int kTM = 64;  // rows (slots) per workgroup
constexpr int kTN = 64;  // output columns per workgroup
constexpr int kTK = 64;  // k chunk
constexpr int kLQ = kTK / 8 + 1;  // padded LDS row stride (uint4)
constexpr int kMaxSplits = 8;     // split-K slices at most

// Split-K partial products: part[ks, m, j] = sum_{k in slice ks} h[m, k] * Wcat[j, k].
// 4 waves as a 2 x 2 grid of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16, layout as in the
// readout kernel: D[row = 8*(v/4) + 4*(l/32) + v%4][col = l%32]). Up to kDepth k chunks are loaded
// into registers ahead of the one being multiplied out of LDS: the operands are first touches
// from HBM, so the slice's loads must be in flight together rather than one chunk at a time.
// The GEMM's own launch takes 8 (10 us at 32 x 16 slots against 25 one chunk at a time); inside
// a start-of-step launch, whose other workgroups need few registers, 4 keeps the launch at four
// workgroups per CU.
struct GemmLds {
  u32x4 a[kTM * kLQ];
  u32x4 b[kTN * kLQ];
};

template <int kDepth>
__device__ __forceinline__ void hidden_gemm_tile(const uint16_t* __restrict__ h,
                                                 const uint16_t* __restrict__ down_h,
                                                 const uint16_t* __restrict__ down_g, int NB,
                                                 int H, int r, int kslice,
                                                 float* __restrict__ part, int bx, int by,
                                                 int ks, GemmLds& lds) {
  u32x4* s_a = lds.a;
  u32x4* s_b = lds.b;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int m0 = bx * kTM, n0 = by * kTN;
  const int kbeg = ks * kslice, kend = min(H, kbeg + kslice);
  const int nch = (kend - kbeg) / kTK;  // H and kslice are multiples of kTK
  const int l32 = lane & 31, half = lane >> 5;
  // this thread's two 16-byte chunks of each k chunk: rows rr0, rr0 + 32 at column cc
  const int rr0 = tid / (kTK / 8), cc = tid % (kTK / 8);
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int rr = rr0 + 32 * q;
    arow[q] = h + (int64_t)min(m0 + rr, NB - 1) * H + kbeg;
    const int j = n0 + rr;  // output column = row of [down_h; down_g]
    brow[q] = ((j < r) ? down_h + (int64_t)j * H : down_g + (int64_t)(j - r) * H) + kbeg;
  }
  // native vectors, not HIP's uint4 struct: struct copies into the slots would keep them in memory
  u32x4 ra[kDepth][2], rb[kDepth][2];
  auto load = [&](auto slotc, int c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slotc)::value;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      ra[slot][q] = reinterpret_cast<const u32x4*>(arow[q] + c * kTK)[cc];
      rb[slot][q] = reinterpret_cast<const u32x4*>(brow[q] + c * kTK)[cc];
    }
  };
  auto stage = [&](auto slotc) __attribute__((always_inline)) {
    constexpr int slot = decltype(slotc)::value;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      s_a[(rr0 + 32 * q) * kLQ + cc] = ra[slot][q];
      s_b[(rr0 + 32 * q) * kLQ + cc] = rb[slot][q];
    }
  };
  f32x16 acc = {};
  auto multiply = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kTK / 16; ++s) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, s_a[(32 * wm + l32) * kLQ + 2 * s + half]);
      const bf16x8 b = __builtin_bit_cast(bf16x8, s_b[(32 * wn + l32) * kLQ + 2 * s + half]);
      acc = mfma32x32x16(a, b, acc);
    }
  };
  // whole groups of kDepth chunks: every load unconditional (the last group's refills repeat its
  // last chunk), so the slots stay in fixed registers
  const int nfull = nch / kDepth * kDepth;
  if (nfull > 0) {
    static_for<0, kDepth>([&](auto dc) __attribute__((always_inline)) {
      load(dc, decltype(dc)::value);
    });
    for (int c0 = 0; c0 < nfull; c0 += kDepth) {
      static_for<0, kDepth>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        stage(dc);
        __syncthreads();
        load(dc, min(c0 + d + kDepth, nfull - 1));
        multiply();
        __syncthreads();
      });
    }
  }
  for (int c = nfull; c < nch; ++c) {  // the rest, one chunk at a time
    load(Int<0>{}, c);
    stage(Int<0>{});
    __syncthreads();
    multiply();
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

}  // namespace

}  // namespace xpress
