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
// Here A = w2 rows (vocabulary ids), B = lat rows (readout rows): D[vocab][row]. Lane l thus
// owns readout row l%32 and, in each group g of 8 ids, the 4 consecutive ids 8g + 4*(l/32) + 0..3.
//
// Work decomposition: a unit is (vocabulary tile of TV = 32*NW ids, 32-row tile). The units are
// numbered vocabulary-tile-major and the persistent grid splits that sequence into equal
// contiguous ranges, so every workgroup scores the same number of row tiles (to within one) and
// reloads its w2 fragment (kept in registers) only when its range crosses into the next
// vocabulary tile.
//
// Data path per unit: the lat tile [32 rows x r] (from L2) and the base tile [32 rows x TV] (from
// HBM) are fetched with fully coalesced 16-byte loads into registers one unit ahead, written to
// a double-buffered, padded LDS stage, and read from there by the MFMA (lat) and by the epilogue
// (base, in the accumulator layout). Coalesced 16-byte loads stream at full HBM rate; reading
// base directly in the accumulator layout (8 bytes per lane, 32 rows per instruction) does not.
//
// Iteration t (one barrier): MFMA + epilogue on stage t%2; write the registers (unit t+1) into
// stage (t+1)%2; issue the loads of unit t+2. Each wave's per-row winners go to a double-buffered
// LDS slot; wave 0 reduces them one unit later and stores the partials. Loads sit outside
// data-dependent branches (rows past the end are clamped to the last row, ids past V to the
// padded row end, which the base stride guarantees is readable), so the compiler's wait counts
// keep them in flight across the iteration.
template <int R, int NW>
__global__ __launch_bounds__(NW * 64) void readout_partial_kernel(
    const uint16_t* __restrict__ lat, const uint16_t* __restrict__ w2,
    const uint16_t* __restrict__ base, int64_t ld, int rows, int V, int ntiles,
    uint2* __restrict__ part, const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int KS = R / 16;
  constexpr int RQ = R / 8;           // 16-byte chunks per lat row
  constexpr int LDQ = RQ + 1;         // padded lat row stride (chunks)
  constexpr int TV = 32 * NW;
  constexpr int BQ = TV / 8;          // 16-byte chunks per base tile row
  constexpr int BLD = BQ + 1;         // padded base row stride (chunks)
  constexpr int NT = NW * 64;
  constexpr int LQ = (32 * RQ + NT - 1) / NT;  // lat chunks per thread
  constexpr int BQT = (32 * BQ + NT - 1) / NT; // base chunks per thread

  __shared__ uint4 s_lat[2][32 * LDQ];
  __shared__ uint4 s_base[2][32 * BLD];
  __shared__ float s_rv[2][NW][32];
  __shared__ int s_ri[2][NW][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int n_rt = (rows + 31) / 32;
  const int64_t units = (int64_t)ntiles * n_rt;
  const int u0 = (int)(units * blockIdx.x / gridDim.x);
  const int u1 = (int)(units * (blockIdx.x + 1) / gridDim.x);
  const int T = u1 - u0;
  if (T <= 0) return;
  const int last_chunk = (V + 7) / 8 - 1;  // last 16-byte chunk inside the padded row

  // Prefetch cursor (unit whose data goes into the staging registers next), kept as
  // (vocabulary tile, row tile) and advanced without divisions; it stops at the last unit.
  int pf_tile = u0 / n_rt, pf_rt = u0 % n_rt, pf_left = T;
  u32x4 lreg[LQ], breg[BQT];
  auto load_next = [&]() __attribute__((always_inline)) {
    const int r0 = pf_rt * 32;
    const int c0 = pf_tile * BQ;
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int idx = min(tid + q * NT, 32 * RQ - 1);
      const int r = min(r0 + idx / RQ, rows - 1);
      lreg[q] = reinterpret_cast<const u32x4*>(lat + (int64_t)r * R)[idx % RQ];
    }
#pragma unroll
    for (int q = 0; q < BQT; ++q) {
      const int idx = min(tid + q * NT, 32 * BQ - 1);
      const int r = min(r0 + idx / BQ, rows - 1);
      const int c = min(c0 + idx % BQ, last_chunk);
      breg[q] = reinterpret_cast<const u32x4*>(base + (int64_t)r * ld)[c];
    }
    if (pf_left > 1) {
      --pf_left;
      if (++pf_rt == n_rt) { pf_rt = 0; ++pf_tile; }
    }
  };
  auto store_staged = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int idx = tid + q * NT;
      if ((32 * RQ) % NT == 0 || idx < 32 * RQ)
        s_lat[buf][(idx / RQ) * LDQ + idx % RQ] =
            make_uint4(lreg[q].x, lreg[q].y, lreg[q].z, lreg[q].w);
    }
#pragma unroll
    for (int q = 0; q < BQT; ++q) {
      const int idx = tid + q * NT;
      if ((32 * BQ) % NT == 0 || idx < 32 * BQ)
        s_base[buf][(idx / BQ) * BLD + idx % BQ] =
            make_uint4(breg[q].x, breg[q].y, breg[q].z, breg[q].w);
    }
  };
  // wave 0: winners of the unit held in s_rv/s_ri[b] across the waves -> global partials.
  // All 64 lanes run it (lanes 32..63 repeat lanes 0..31 and store the same values).
  auto flush = [&](int b, int tile, int rt) __attribute__((always_inline)) {
    float v = s_rv[b][0][l32];
    int i = s_ri[b][0][l32];
#pragma unroll
    for (int w = 1; w < NW; ++w) argmax_merge(v, i, s_rv[b][w][l32], s_ri[b][w][l32]);
    const int prow = rt * 32 + l32;
    if (prow < rows) part[(int64_t)prow * ntiles + tile] = make_uint2(__float_as_uint(v), (unsigned)i);
  };

  load_next();
  store_staged(0);
  load_next();
  __syncthreads();

  int t = 0;
  int tile = u0 / n_rt, rt = u0 % n_rt;
  int prev_tile = 0, prev_rt = 0;
  bf16x8 a[KS];
  while (t < T) {
    // segment: the units of this workgroup's range that share vocabulary tile `tile`
    const int seg_end = min(T, t + (n_rt - rt));
    {
      const int v = min(tile * TV + wave * 32 + l32, V - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(w2 + (int64_t)v * R) + half;
#pragma unroll
      for (int s = 0; s < KS; ++s) a[s] = __builtin_bit_cast(bf16x8, src[2 * s]);
    }
    const int vl = tile * TV + wave * 32 + 4 * half;
    const bool full_tile = (tile + 1) * TV <= V;
    for (; t < seg_end; ++t, ++rt) {
      const int buf = t & 1;
      f32x16 acc = {};
      const uint4* sl = s_lat[buf];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = mfma32x32x16(a[s], as_bf16x8(sl[l32 * LDQ + 2 * s + half]), acc);
      // this lane's base values: row l32, ids 32*wave + 8g + 4*half + 0..3 of the tile
      const uint2* sb = reinterpret_cast<const uint2*>(s_base[buf] + l32 * BLD + wave * 4);
      float lg[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 q = sb[2 * g + half];
        lg[4 * g + 0] = acc[4 * g + 0] + bf16_lo(q.x);
        lg[4 * g + 1] = acc[4 * g + 1] + bf16_hi(q.x);
        lg[4 * g + 2] = acc[4 * g + 2] + bf16_lo(q.y);
        lg[4 * g + 3] = acc[4 * g + 3] + bf16_hi(q.y);
      }
      float bv = lg[0];
      int bl = 0;  // local index 4g + k of this lane's best id
      if (full_tile) {
#pragma unroll
        for (int e = 1; e < 16; ++e) {
          const bool gt = lg[e] > bv;
          bv = gt ? lg[e] : bv;
          bl = gt ? e : bl;
        }
      } else {  // the tile straddling V: ids >= V never win
        bv = (vl < V) ? lg[0] : -INFINITY;
#pragma unroll
        for (int e = 1; e < 16; ++e) {
          const bool gt = (vl + 8 * (e >> 2) + (e & 3) < V) & (lg[e] > bv);
          bv = gt ? lg[e] : bv;
          bl = gt ? e : bl;
        }
      }
      int bi = vl + 8 * (bl >> 2) + (bl & 3);
      {
        const float ov = __shfl_xor(bv, 32);
        const int oi = __shfl_xor(bi, 32);
        argmax_merge(bv, bi, ov, oi);
      }
      if (lane < 32) {
        s_rv[buf][wave][lane] = bv;
        s_ri[buf][wave][lane] = bi;
      }
      if (t > 0 && wave == 0) flush(buf ^ 1, prev_tile, prev_rt);
      store_staged(buf ^ 1);
      load_next();
      prev_tile = tile;
      prev_rt = rt;
      __syncthreads();
    }
    ++tile;
    rt = 0;
  }
  if (wave == 0) flush((T - 1) & 1, prev_tile, prev_rt);
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

template <int R, int NW>
hipError_t launch_partial_t(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                            int64_t ld, int rows, int64_t V, uint2* part, const int32_t* flags,
                            int pass, hipStream_t s) {
  const int ntiles = readout_tiles(V);
  const int64_t units = (int64_t)ntiles * ((rows + 31) / 32);
  int64_t grid = (int64_t)device_cus() * readout_wgs_per_cu();
  if (grid > units) grid = units;
  hipLaunchKernelGGL((readout_partial_kernel<R, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s,
                     lat, w2, base, ld, rows, (int)V, ntiles, part, flags, pass);
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

int readout_wgs_per_cu() {
  static const int n = env_int("XPRESS_READOUT_WGS_PER_CU", 1);
  return n;
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
