// Full-vocabulary readout + argmax of one XPress pass (gfx950).
//
// Computes, for every readout row p and vocabulary id v,
//   logit[p, v] = base[p, v] + sum_c lat[p, c] * w2[v, c]
// and blk[n, 1 + p % (B-1)] = argmax_v logit[p, v] (lowest id on ties), without ever storing the
// [rows, V] logits (vLLM API page "vllm.v1.worker.gpu.spec_decode.xpress.kernels": module
// docstring's readout and argmax stages, fused_add_argmax_to_blk).
//
// K5 (readout_partial_kernel) is a bf16 MFMA GEMM, lat [rows, r] x w2^T [r, V], whose epilogue
// adds the bf16 base tile to the fp32 accumulators and reduces each row to one (max, lowest id)
// pair per vocabulary tile. Each wave keeps the w2 fragment of its 32 vocabulary ids in registers
// for the whole launch (w2 crosses HBM once per pass), streams 32-row tiles of lat through LDS
// (shared by the workgroup's waves) and reads base straight from HBM in the accumulator layout.
// K6 (argmax_reduce_kernel) reduces a row's tile partials and writes the winner into blk in place.
#include "launch.hpp"
#include "xpress_common.hpp"

#include <limits.h>
#include <stdlib.h>

namespace xpress {

namespace {

constexpr int kReadoutWavesDefault = 8;

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  int v = atoi(s);
  return v > 0 ? v : dflt;
}

// v_mfma_f32_32x32x16_bf16 operand layout (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + e, e = 0..7
//   B (16 x 32): lane l holds col l%32, the same k
//   D (32 x 32): lane l, accumulator v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// Here A = w2 rows (vocabulary ids), B = lat rows (readout rows): D[vocab][row].
template <int R, int NW>
__global__ __launch_bounds__(NW * 64) void readout_partial_kernel(
    const uint16_t* __restrict__ lat, const uint16_t* __restrict__ w2,
    const uint16_t* __restrict__ base, int64_t ld, int rows, int V, int ntiles, int row_groups,
    uint2* __restrict__ part, const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int KS = R / 16;       // MFMA k-steps
  constexpr int RQ = R / 8;        // uint4 (8 x bf16) per lat / w2 row
  constexpr int LDQ = RQ + 1;      // padded LDS row stride in uint4
  constexpr int TV = 32 * NW;      // vocabulary ids per workgroup

  __shared__ uint4 s_lat[32 * LDQ];
  __shared__ float s_rv[NW][32];
  __shared__ int s_ri[NW][32];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // XCD-aware mapping: workgroup ids are dealt round-robin to the 8 XCDs, so the row groups of
  // one vocabulary tile get ids 8 apart and share an XCD (and its L2 copy of the w2 tile).
  const int wg = blockIdx.x;
  const int grp = wg / (8 * row_groups);
  const int within = wg % (8 * row_groups);
  const int tile = grp * 8 + (within & 7);
  const int rg = within >> 3;
  if (tile >= ntiles) return;

  const int v0 = tile * TV + wave * 32;
  const bool wave_live = v0 < V;

  bf16x8 a[KS];
  {
    const int v = v0 + l32;
    if (v < V) {
      const uint4* src = reinterpret_cast<const uint4*>(w2 + (int64_t)v * R) + half;
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = as_bf16x8(ld_nt16(src + 2 * s));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  const bool tail_tile = (tile + 1) * TV > V;
  const int n_rt = (rows + 31) / 32;

  for (int rt = rg; rt < n_rt; rt += row_groups) {
    const int r0 = rt * 32;
    for (int q = threadIdx.x; q < 32 * RQ; q += NW * 64) {
      const int rr = q / RQ, cc = q % RQ;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r0 + rr < rows) val = reinterpret_cast<const uint4*>(lat + (int64_t)(r0 + rr) * R)[cc];
      s_lat[rr * LDQ + cc] = val;
    }
    __syncthreads();

    float bv = -INFINITY;
    int bi = INT_MAX;
    const int row = r0 + l32;
    if (wave_live) {
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 b = as_bf16x8(s_lat[l32 * LDQ + 2 * s + half]);
        acc = mfma32x32x16(a[s], b, acc);
      }
      if (row < rows) {
        const uint16_t* brow = base + (int64_t)row * ld;
        const int vl = v0 + 4 * half;  // this lane's first id in each group of 8
        if (!tail_tile) {
          uint2 q[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            q[g] = ld_nt8(brow + vl + 8 * g);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float l0 = acc[4 * g + 0] + bf16_lo(q[g].x);
            const float l1 = acc[4 * g + 1] + bf16_hi(q[g].x);
            const float l2 = acc[4 * g + 2] + bf16_lo(q[g].y);
            const float l3 = acc[4 * g + 3] + bf16_hi(q[g].y);
            const int id = vl + 8 * g;
            if (l0 > bv) { bv = l0; bi = id; }
            if (l1 > bv) { bv = l1; bi = id + 1; }
            if (l2 > bv) { bv = l2; bi = id + 2; }
            if (l3 > bv) { bv = l3; bi = id + 3; }
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int id = vl + 8 * g + e;
              if (id < V) {
                const float l = acc[4 * g + e] + bf16_to_f32(brow[id]);
                if (l > bv) { bv = l; bi = id; }
              }
            }
        }
      }
    }
    // lanes l and l^32 hold the two interleaved halves of the same row
    {
      const float ov = __shfl_xor(bv, 32);
      const int oi = __shfl_xor(bi, 32);
      argmax_merge(bv, bi, ov, oi);
    }
    if (lane < 32) {
      s_rv[wave][lane] = bv;
      s_ri[wave][lane] = bi;
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      float v = s_rv[0][threadIdx.x];
      int i = s_ri[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < NW; ++w) argmax_merge(v, i, s_rv[w][threadIdx.x], s_ri[w][threadIdx.x]);
      const int prow = r0 + threadIdx.x;
      if (prow < rows) part[(int64_t)prow * ntiles + tile] = make_uint2(__float_as_uint(v), (unsigned)i);
    }
  }
}

// One workgroup per readout row: reduce the row's tile partials, write blk in place, flag changes.
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

template <int R, int NW>
hipError_t launch_partial_t(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                            int64_t ld, int rows, int64_t V, uint2* part, const int32_t* flags,
                            int pass, hipStream_t s) {
  const int ntiles = readout_tiles(V);
  const int rg = readout_row_groups(rows, V);
  const int groups = (ntiles + 7) / 8;
  dim3 grid(groups * 8 * rg), block(NW * 64);
  hipLaunchKernelGGL((readout_partial_kernel<R, NW>), grid, block, 0, s, lat, w2, base, ld, rows,
                     (int)V, ntiles, rg, part, flags, pass);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_partial_nw(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                             int64_t ld, int rows, int64_t V, int r, uint2* part,
                             const int32_t* flags, int pass, hipStream_t s) {
  switch (r) {
    case 64: return launch_partial_t<64, NW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    case 128: return launch_partial_t<128, NW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    case 256: return launch_partial_t<256, NW>(lat, w2, base, ld, rows, V, part, flags, pass, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int readout_waves() {
  static const int nw = [] {
    int v = env_int("XPRESS_READOUT_WAVES", kReadoutWavesDefault);
    return (v == 4 || v == 8 || v == 16) ? v : kReadoutWavesDefault;
  }();
  return nw;
}

int readout_tiles(int64_t V) {
  const int64_t tv = 32 * readout_waves();
  return (int)((V + tv - 1) / tv);
}

int readout_row_groups(int rows, int64_t V) {
  const int n_rt = (rows + 31) / 32;
  const int forced = env_int("XPRESS_READOUT_ROW_GROUPS", 0);
  int rg = forced > 0 ? forced : (1024 + readout_tiles(V) - 1) / readout_tiles(V);
  if (rg > n_rt) rg = n_rt;
  return rg < 1 ? 1 : rg;
}

hipError_t launch_readout_partial(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                                  int64_t ld, int rows, int64_t V, int r, uint2* part,
                                  const int32_t* flags, int pass, hipStream_t s) {
  switch (readout_waves()) {
    case 4: return launch_partial_nw<4>(lat, w2, base, ld, rows, V, r, part, flags, pass, s);
    case 16: return launch_partial_nw<16>(lat, w2, base, ld, rows, V, r, part, flags, pass, s);
    default: return launch_partial_nw<8>(lat, w2, base, ld, rows, V, r, part, flags, pass, s);
  }
}

hipError_t launch_argmax_reduce(const uint2* part, int ntiles, int rows, int B, int64_t* blk,
                                int32_t* changed, int32_t* flags, int pass, hipStream_t s) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(rows), dim3(256), 0, s, part, ntiles, rows, B,
                     blk, changed, flags, pass);
  return hipGetLastError();
}

}  // namespace xpress
