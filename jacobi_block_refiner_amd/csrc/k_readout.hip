// Full-vocabulary readout + argmax of one XPress pass (gfx950).
//
// Computes, for every readout row p and vocabulary id v,
//   logit[p, v] = base[p, v] + sum_c lat[p, c] * w2[v, c]
// and blk[n, 1 + p % (B-1)] = argmax_v logit[p, v] (lowest id on ties), without ever storing the
// [rows, V] logits (vLLM API page "vllm.v1.worker.gpu.spec_decode.xpress.kernels": module
// docstring's readout and argmax stages, fused_add_argmax_to_blk).
//
// K5 (readout_partial_kernel) is a bf16 MFMA GEMM, lat [rows, r] x w2^T [r, V], whose epilogue
// adds the bf16 base tile to the fp32 accumulators and keeps a running (max, lowest id) per row.
// K6 (argmax_reduce_kernel) reduces a row's partials and writes the winner into blk in place.
//
// K5 is lat-stationary. The readout rows are few (tens to a few hundred) and lat is tiny, while
// w2 and base stream from HBM once per pass. A workgroup owns a chunk of up to 8*RW 32-row tiles
// and a contiguous range of 32-id vocabulary steps; each of its 8 waves keeps the lat fragments
// of its RW row tiles in registers for the whole launch. Per step, the w2 tile [32 ids x r] and
// the base tile [chunk rows x 32 ids] are fetched with coalesced 16-byte loads into registers
// one step ahead, written into a double-buffered LDS stage, and every wave multiplies the shared
// w2 tile against its own rows. Each w2 fragment read from LDS feeds RW MFMAs, and the per-row
// winners stay in registers across the whole range: one partial per (row, range) is written at
// the end. The ranges of one row chunk split the vocabulary evenly over the workgroups.
#include "launch.hpp"
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

namespace {

constexpr int kNW = 8;              // waves per workgroup
constexpr int kNT = 64 * kNW;       // threads per workgroup
constexpr int kMaxRanges = 256;     // vocabulary ranges per row chunk (partials per row)
constexpr int kBaseUnits = 9;       // 8-byte LDS units per base row of a step (64 bytes + pad)

// v_mfma_f32_32x32x16_bf16 operand layout (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + e, e = 0..7
//   B (16 x 32): lane l holds col l%32, the same k
//   D (32 x 32): lane l, accumulator v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// Here A = w2 rows (vocabulary ids), B = lat rows (readout rows): D[vocab][row]. Lane l thus
// owns readout row l%32 and, in each group g of 8 ids of a step, the 4 consecutive ids
// 8g + 4*(l/32) + 0..3, which it visits in increasing id order.
//
// LDS layouts. w2 tile: id i's 16-byte chunk c sits at i*RQ + (c ^ (i % RQ)), so the 16 lanes of
// an A-fragment read (16 ids, one chunk) hit 16 different bank groups. base tile: row stride of
// 72 bytes, so the 8-byte reads of 32 rows (one per lane) spread over all banks.
template <int R, int RW>
__global__ __launch_bounds__(kNT) void readout_partial_kernel(
    const uint16_t* __restrict__ lat, const uint16_t* __restrict__ w2,
    const uint16_t* __restrict__ base, int64_t ld, int rows, int V, int nvr, int n_rc,
    uint2* __restrict__ part, const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int KS = R / 16;
  constexpr int RQ = R / 8;                        // 16-byte chunks per w2 / lat row
  constexpr int CH = kNW * RW * 32;                // rows per row chunk
  constexpr int WQ = (32 * RQ + kNT - 1) / kNT;    // w2 chunks per thread per step
  constexpr int BQ = CH * 4 / kNT;                 // base chunks per thread per step

  __shared__ uint4 s_w2[2][32 * RQ];
  __shared__ uint2 s_base[2][CH * kBaseUnits];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // (row chunk, vocabulary range) of this workgroup. With several row chunks and ranges in
  // multiples of 8, the chunks of one range go to workgroups on the same XCD (workgroups are
  // dealt round-robin over the 8 XCDs), so its w2 tiles are fetched into that XCD's L2 once.
  int rc, vr;
  if (n_rc == 1) {
    rc = 0;
    vr = blockIdx.x;
  } else if ((nvr & 7) == 0) {
    const int j = blockIdx.x >> 3;
    rc = j % n_rc;
    vr = (j / n_rc) * 8 + (blockIdx.x & 7);
  } else {
    rc = blockIdx.x / nvr;
    vr = blockIdx.x % nvr;
  }
  const int nsteps = (V + 31) / 32;
  const int t0 = (int)((int64_t)nsteps * vr / nvr);
  const int t1 = (int)((int64_t)nsteps * (vr + 1) / nvr);
  if (t1 <= t0) return;
  const int row0 = rc * CH;
  const int last_chunk = (V + 7) / 8 - 1;  // last 16-byte chunk inside the padded base row

  // lat fragments (B operand) of this wave's row tiles, held for the whole launch
  bf16x8 bl[RW][KS];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    const int row = min(row0 + (wave * RW + k) * 32 + l32, rows - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(lat + (int64_t)row * R);
#pragma unroll
    for (int s = 0; s < KS; ++s) bl[k][s] = __builtin_bit_cast(bf16x8, src[2 * s + half]);
  }
  const bool active = row0 + wave * RW * 32 < rows;  // wave-uniform: the wave has real rows

  // staging registers: the next step's w2 and base chunks
  u32x4 wreg[WQ], breg[BQ];
  auto load_step = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int q = min(tid + i * kNT, 32 * RQ - 1);
      const int v = min(32 * t + q / RQ, V - 1);
      wreg[i] = reinterpret_cast<const u32x4*>(w2 + (int64_t)v * R)[q % RQ];
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int q = tid + i * kNT;
      const int r = min(row0 + (q >> 2), rows - 1);
      breg[i] = reinterpret_cast<const u32x4*>(base + (int64_t)r * ld)[min(4 * t + (q & 3), last_chunk)];
    }
  };
  // Registers -> LDS stage. Base values of ids >= V (the padding of the last chunk, and chunks
  // past V in the last step) become -inf, so they never win.
  auto store_step = [&](int buf, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int q = tid + i * kNT;
      if ((32 * RQ) % kNT == 0 || q < 32 * RQ) {
        const int id = q / RQ, c = q % RQ;
        s_w2[buf][id * RQ + (c ^ (id % RQ))] = make_uint4(wreg[i].x, wreg[i].y, wreg[i].z, wreg[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < BQ; ++i) {
      const int q = tid + i * kNT;
      const int id0 = 32 * t + 8 * (q & 3);
      u32x4 v = breg[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (id0 + 2 * e < V) ? (v[e] & 0xffffu) : 0xff80u;
        const uint32_t hi = (id0 + 2 * e + 1 < V) ? (v[e] >> 16) : 0xff80u;
        v[e] = lo | (hi << 16);
      }
      uint2* d = &s_base[buf][(q >> 2) * kBaseUnits + 2 * (q & 3)];
      d[0] = make_uint2(v.x, v.y);
      d[1] = make_uint2(v.z, v.w);
    }
  };

  float bv[RW];
  int bi[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    bv[k] = -INFINITY;
    bi[k] = 32 * t0;
  }
  // Step t of row tile k: logits of this lane's row for its 16 ids of the step, folded into
  // the running winner. Within the step the ids rise with e, and steps rise with t, so a strict
  // comparison keeps the lowest id among equal values.
  auto epilogue = [&](int buf, int t, int k, const f32x16& acc) __attribute__((always_inline)) {
    const uint2* sb = &s_base[buf][((wave * RW + k) * 32 + l32) * kBaseUnits + half];
    float lg[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 q = sb[2 * g];
      lg[4 * g + 0] = acc[4 * g + 0] + bf16_lo(q.x);
      lg[4 * g + 1] = acc[4 * g + 1] + bf16_hi(q.x);
      lg[4 * g + 2] = acc[4 * g + 2] + bf16_lo(q.y);
      lg[4 * g + 3] = acc[4 * g + 3] + bf16_hi(q.y);
    }
    float sv = lg[0];
    int se = 0;
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      const bool gt = lg[e] > sv;
      sv = gt ? lg[e] : sv;
      se = gt ? e : se;
    }
    const bool gt = sv > bv[k];
    bv[k] = gt ? sv : bv[k];
    bi[k] = gt ? 32 * t + 4 * half + 8 * (se >> 2) + (se & 3) : bi[k];
  };

  // prologue: stage 0 <- step t0, registers <- step t0+1
  load_step(t0);
  store_step(0, t0);
  load_step(min(t0 + 1, t1 - 1));
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    if (active) {
      f32x16 acc[RW];
#pragma unroll
      for (int k = 0; k < RW; ++k) acc[k] = f32x16{};
      const uint4* sw = s_w2[buf] + l32 * RQ;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = as_bf16x8(sw[(2 * s + half) ^ (l32 % RQ)]);
#pragma unroll
        for (int k = 0; k < RW; ++k) acc[k] = mfma32x32x16(a, bl[k][s], acc[k]);
      }
#pragma unroll
      for (int k = 0; k < RW; ++k) epilogue(buf, t, k, acc[k]);
    }
    // stage buf^1 was last read in the previous step, before its barrier
    store_step(buf ^ 1, min(t + 1, t1 - 1));
    load_step(min(t + 2, t1 - 1));  // past the range end: reloads the last step (L2 hits)
    __syncthreads();
  }

  // lanes l and l^32 hold the same row with interleaved ids
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    float v = bv[k];
    int i = bi[k];
    const float ov = __shfl_xor(v, 32);
    const int oi = __shfl_xor(i, 32);
    argmax_merge(v, i, ov, oi);
    const int row = row0 + (wave * RW + k) * 32 + l32;
    if (half == 0 && row < rows) part[(int64_t)row * nvr + vr] = make_uint2(__float_as_uint(v), (unsigned)i);
  }
}

// One workgroup per readout row: reduce the row's range partials, write blk in place, flag changes.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const uint2* __restrict__ part,
                                                            int ntiles, int rows, int B,
                                                            int64_t* __restrict__ blk,
                                                            int32_t* changed, int32_t* flags,
                                                            int pass) {
  if (pass_skipped(flags, pass)) return;
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int p = blockIdx.x;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const uint2* pr = part + (int64_t)p * ntiles;
  for (int t = threadIdx.x; t < ntiles; t += 256) {
    const uint2 q = pr[t];
    argmax_merge(bv, bi, __uint_as_float(q.x), (int)q.y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    argmax_merge(bv, bi, ov, oi);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, s_v[w], s_i[w]);
    const int n = p / (B - 1), b = 1 + p % (B - 1);
    int64_t* slot = blk + (int64_t)n * B + b;
    const int64_t nv = (int64_t)bi;
    if (*slot != nv) {
      *slot = nv;
      if (changed) __hip_atomic_store(changed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (flags) __hip_atomic_store(flags + pass, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int device_cus() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

template <int R, int RW>
hipError_t launch_partial_t(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                            int64_t ld, int rows, int64_t V, uint2* part, const int32_t* flags,
                            int pass, hipStream_t s) {
  const int nvr = readout_tiles(V);
  constexpr int CH = kNW * RW * 32;
  const int n_rc = (rows + CH - 1) / CH;
  hipLaunchKernelGGL((readout_partial_kernel<R, RW>), dim3((unsigned)(nvr * n_rc)), dim3(kNT), 0, s,
                     lat, w2, base, ld, rows, (int)V, nvr, n_rc, part, flags, pass);
  return hipGetLastError();
}

template <int RW>
hipError_t launch_partial_rw(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                             int64_t ld, int rows, int64_t V, int r, uint2* part,
                             const int32_t* flags, int pass, hipStream_t s) {
  switch (r) {
    case 64: return launch_partial_t<64, RW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    case 128: return launch_partial_t<128, RW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    case 256: return launch_partial_t<256, RW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int readout_tiles(int64_t V) {
  const int64_t steps = (V + 31) / 32;
  return (int)(steps < kMaxRanges ? steps : kMaxRanges);
}

hipError_t launch_readout_partial(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                                  int64_t ld, int rows, int64_t V, int r, uint2* part,
                                  const int32_t* flags, int pass, hipStream_t s) {
  if (rows <= kNW * 32) return launch_partial_rw<1>(lat, w2, base, ld, rows, V, r, part, flags, pass, s);
  return launch_partial_rw<2>(lat, w2, base, ld, rows, V, r, part, flags, pass, s);
}

hipError_t launch_argmax_reduce(const uint2* part, int ntiles, int rows, int B, int64_t* blk,
                                int32_t* changed, int32_t* flags, int pass, hipStream_t s) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(rows), dim3(256), 0, s, part, ntiles, rows, B,
                     blk, changed, flags, pass);
  return hipGetLastError();
}

}  // namespace xpress
