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
// Iteration t (one barrier) is software-pipelined: the MFMA chain of unit t+1 (into a second
// accumulator, with unit t+1's base values read from LDS into registers) and the epilogue of unit t
// form one branch-free block, so the VALU can work on unit t while the matrix core works on
// unit t+1; then the register set holding
// unit t+2 is written into the freed LDS stage and refilled with the loads of unit t+4 (two
// register sets alternate, so every load has two iterations to arrive). Each wave's
// per-row winners go to a double-buffered LDS slot; wave 0 reduces them one unit later and stores
// the partials. Loads sit outside data-dependent branches (rows past the end are clamped to the
// last row, ids past V to the padded row end, which the base stride guarantees is readable), so
// the compiler's wait counts keep them in flight across the iteration.
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
  // two register sets: loads run two iterations ahead; set_tile[k] is the vocabulary tile of the
  // unit held in set k
  u32x4 lreg_s[2][LQ], breg_s[2][BQT];
  int set_tile[2];
  auto load_next = [&](u32x4 (&lreg)[LQ], u32x4 (&breg)[BQT], int& stile) __attribute__((always_inline)) {
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
      breg[q] = reinterpret_cast<const u32x4*>(base + (int64_t)r * ld)[min(c0 + idx % BQ, last_chunk)];
    }
    stile = pf_tile;
    if (pf_left > 1) {
      --pf_left;
      if (++pf_rt == n_rt) { pf_rt = 0; ++pf_tile; }
    }
  };
  // Register set -> LDS stage. Base values of ids >= V (the padding of the last chunk, and chunks
  // past V in the tile that straddles V) become -inf, so they never win and the epilogue needs no
  // bound check. The masking runs here, where the loaded values are consumed anyway, not right
  // after the loads (which would wait for them).
  auto store_staged = [&](int buf, const u32x4 (&lreg)[LQ], const u32x4 (&breg)[BQT], int stile) __attribute__((always_inline)) {
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
      const int id0 = 8 * (stile * BQ + idx % BQ);
      u32x4 v = breg[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (id0 + 2 * e < V) ? (v[e] & 0xffffu) : 0xff80u;
        const uint32_t hi = (id0 + 2 * e + 1 < V) ? (v[e] >> 16) : 0xff80u;
        v[e] = lo | (hi << 16);
      }
      if ((32 * BQ) % NT == 0 || idx < 32 * BQ)
        s_base[buf][(idx / BQ) * BLD + idx % BQ] = make_uint4(v.x, v.y, v.z, v.w);
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

  bf16x8 a[KS];
  int cur_tile = -1;
  auto load_w2 = [&](int tile) __attribute__((always_inline)) {
    const int v = min(tile * TV + wave * 32 + l32, V - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(w2 + (int64_t)v * R) + half;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[s] = __builtin_bit_cast(bf16x8, src[2 * s]);
    // Wait for these loads here, in the (rare) tile-change branch. Otherwise the MFMA chain,
    // which is shared by both paths, would carry a conservative wait for every load in flight
    // (vmcnt 0) on every unit and defeat the prefetch of the staged units.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt untouched
    cur_tile = tile;
  };
  auto mfma_unit = [&](int buf, f32x16& acc, uint2 (&bq)[4]) __attribute__((always_inline)) {
    acc = f32x16{};
    const uint4* sl = s_lat[buf];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = mfma32x32x16(a[s], as_bf16x8(sl[l32 * LDQ + 2 * s + half]), acc);
    // this lane's base values: row l32, ids 32*wave + 8g + 4*half + 0..3 of the tile
    const uint2* sb = reinterpret_cast<const uint2*>(s_base[buf] + l32 * BLD + wave * 4);
#pragma unroll
    for (int g = 0; g < 4; ++g) bq[g] = sb[2 * g + half];
  };
  auto epilogue = [&](int t, int tile, const f32x16& acc, const uint2 (&bq)[4]) __attribute__((always_inline)) {
    float lg[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      lg[4 * g + 0] = acc[4 * g + 0] + bf16_lo(bq[g].x);
      lg[4 * g + 1] = acc[4 * g + 1] + bf16_hi(bq[g].x);
      lg[4 * g + 2] = acc[4 * g + 2] + bf16_lo(bq[g].y);
      lg[4 * g + 3] = acc[4 * g + 3] + bf16_hi(bq[g].y);
    }
    const int vl = tile * TV + wave * 32 + 4 * half;
    float bv = lg[0];
    int bl = 0;  // local index 4g + k of this lane's best id
#pragma unroll
    for (int e = 1; e < 16; ++e) {
      const bool gt = lg[e] > bv;
      bv = gt ? lg[e] : bv;
      bl = gt ? e : bl;
    }
    int bi = vl + 8 * (bl >> 2) + (bl & 3);
    const float ov = __shfl_xor(bv, 32);
    const int oi = __shfl_xor(bi, 32);
    argmax_merge(bv, bi, ov, oi);
    // lanes l and l^32 now hold the same winner: both write it (same address, same value)
    s_rv[t & 1][wave][l32] = bv;
    s_ri[t & 1][wave][l32] = bi;
  };

  // prologue: stage 0 <- unit 0, stage 1 <- unit 1, register sets <- units 2 and 3,
  // acc <- unit 0
  load_next(lreg_s[0], breg_s[0], set_tile[0]);
  store_staged(0, lreg_s[0], breg_s[0], set_tile[0]);
  load_next(lreg_s[1], breg_s[1], set_tile[1]);
  store_staged(1, lreg_s[1], breg_s[1], set_tile[1]);
  load_next(lreg_s[0], breg_s[0], set_tile[0]);
  load_next(lreg_s[1], breg_s[1], set_tile[1]);
  __syncthreads();
  int tile = u0 / n_rt, rt = u0 % n_rt;  // unit t
  int ntile = tile, nrt = rt;            // unit t+1
  if (++nrt == n_rt) { nrt = 0; ++ntile; }
  int ptile = 0, prt = 0;                // unit t-1
  f32x16 acc0, acc1;
  uint2 bq0[4], bq1[4];
  load_w2(tile);
  mfma_unit(0, acc0, bq0);
  __syncthreads();  // stage 0 is rewritten (unit 2) in the first iteration

  auto iter = [&](int t, f32x16& acc_cur, uint2 (&bq_cur)[4], f32x16& acc_nxt,
                  uint2 (&bq_nxt)[4], u32x4 (&lreg)[LQ], u32x4 (&breg)[BQT], int& stile)
                  __attribute__((always_inline)) {
    if (ntile != cur_tile) load_w2(ntile);  // workgroup-uniform, rare
    mfma_unit((t + 1) & 1, acc_nxt, bq_nxt);  // past the last unit: recomputes a staged unit
    epilogue(t, tile, acc_cur, bq_cur);
    if (t > 0 && wave == 0) flush((t - 1) & 1, ptile, prt);
    // stage t%2 (unit t) was last read by the MFMA and base reads of the previous iteration,
    // which every wave finished before that iteration's barrier
    store_staged(t & 1, lreg, breg, stile);  // unit t+2 (register set t%2)
    load_next(lreg, breg, stile);            // unit t+4
    __syncthreads();
    ptile = tile; prt = rt;
    tile = ntile; rt = nrt;
    if (++nrt == n_rt) { nrt = 0; ++ntile; }
  };
  int t = 0;
  for (; t + 1 < T; t += 2) {
    iter(t, acc0, bq0, acc1, bq1, lreg_s[0], breg_s[0], set_tile[0]);
    iter(t + 1, acc1, bq1, acc0, bq0, lreg_s[1], breg_s[1], set_tile[1]);
  }
  if (t < T) iter(t, acc0, bq0, acc1, bq1, lreg_s[0], breg_s[0], set_tile[0]);
  if (wave == 0) flush((T - 1) & 1, ptile, prt);
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
