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
// the base tile [chunk rows x 32 ids] are copied from HBM straight into LDS by the load units
// (global_load_lds_dwordx4: no registers, no VALU), into a ring of three stages, so two steps are
// in flight while one is computed. Every wave multiplies the shared w2 tile against its own rows;
// each w2 fragment read from LDS feeds RW MFMAs, and the per-row winners stay in registers across
// the whole range: one partial per (row, range) is written at the end.
#include "launch.hpp"
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

namespace {

constexpr int kMaxRanges = 256;     // vocabulary ranges per row chunk (partials per row)

// v_mfma_f32_32x32x16_bf16 operand layout (wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) + e, e = 0..7
//   B (16 x 32): lane l holds col l%32, the same k
//   D (32 x 32): lane l, accumulator v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// Here A = w2 rows, B = lat rows: D[vocab][row]. A-row i of a step holds vocabulary id
// 16*((i/4)%2) + 4*(i/8) + i%4 of the step, so that lane l, accumulator v scores readout row l%32
// against id 16*(l/32) + v: each lane owns 16 consecutive ids of its row (two 16-byte base chunks)
// and visits them in increasing order.
//
// LDS stage layout (16-byte chunks). w2: the tile is written by RQ/2 copy instructions of 64
// chunks each (RPI = 64/RQ whole w2 rows per instruction), placed 65 chunks apart (one pad
// chunk), and A-row i sits in instruction i % (RQ/2), sub-row i / (RQ/2). Lane l then reads
// fragment s at a per-lane base plus the immediate 32*s bytes (no address arithmetic in the
// loop), and at r = 256 the 16 lanes of a read phase hit 16 different bank groups. base: row rr,
// chunk c at 4*rr + (c ^ ((rr / 4) % 4)) (XOR swizzle). The copy engine writes lane j of a
// global_load_lds_dwordx4 to M0 + 16*j, so each copy instruction fills 64 consecutive chunks and
// its lanes fetch whichever global chunks belong there.
__device__ __forceinline__ int w2_row_id(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <int R, int kNW, int RW, int NS, int TR>
__global__ __launch_bounds__(64 * kNW) void readout_partial_kernel(
    const uint16_t* __restrict__ lat, const uint16_t* __restrict__ w2,
    const uint16_t* __restrict__ base, int64_t ld, int rows, int V, int nvr, int n_rc,
    uint2* __restrict__ part, const int32_t* __restrict__ flags, int pass, int lat_frag) {
  if (pass_skipped(flags, pass)) return;
  constexpr int KS = R / 16;
  constexpr int RQ = R / 8;                     // 16-byte chunks per w2 / lat row
  constexpr int RPI = 64 / RQ;                  // w2 rows per copy instruction
  constexpr int NI = 32 / RPI;                  // copy instructions per w2 tile
  constexpr int WP = 65;                        // chunks per w2 copy block (64 + pad)
  static_assert(TR >= 1 && TR <= kNW * RW, "row tiles per chunk");
  constexpr int CH = TR * 32;                   // rows per row chunk (waves past TR/RW only copy)
  constexpr int WCH = NI * WP;                  // w2 chunks per stage
  constexpr int BCH = CH * 4;                   // base chunks per stage
  constexpr int SCH = WCH + BCH;                // chunks per stage
  // copy instructions per wave per step; when the w2 tile has fewer than kNW instructions, the
  // waves past them repeat the first ones (same bytes to the same place), so every wave issues
  // the same number of copies and one vmcnt value fits all
  constexpr int WI = (NI + kNW - 1) / kNW;
  // base copy instructions per stage, and per wave (as for w2, waves past them repeat the first)
  constexpr int NBI = BCH / 64;
  constexpr int BI = (NBI + kNW - 1) / kNW;
  constexpr int DI = WI + BI;

  __shared__ uint4 s_stage[NS][SCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int rc, vr;
  if (n_rc == 1) {
    rc = 0;
    vr = blockIdx.x;
  } else if ((nvr & 7) == 0) {
    // the row chunks of one range on one XCD (workgroups are dealt round-robin over the 8
    // XCDs), so its w2 tiles reach that XCD's L2 once
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

  // lat fragments (B operand) of this wave's row tiles, held for the whole launch. From a
  // row-major lat each load instruction touches 32 rows; in a step, lat is in fragment order
  // (lat_frag_offset) and each instruction reads 1 KiB contiguous (every workgroup loads all its
  // chunk's rows, 256 KB at 512 rows: 44.6 against 49.8 us per readout at 480 rows). Tiles past
  // the last real row repeat it; their rows are never written out.
  bf16x8 bl[RW][KS];
  if (lat_frag) {
    const int last_tile = (rows - 1) >> 5;
#pragma unroll
    for (int k = 0; k < RW; ++k) {
      const int T = min((row0 >> 5) + wave * RW + k, last_tile);
      const u32x4* src = reinterpret_cast<const u32x4*>(lat) + (int64_t)T * KS * 64 + lane;
#pragma unroll
      for (int s = 0; s < KS; ++s) bl[k][s] = __builtin_bit_cast(bf16x8, src[s * 64]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < RW; ++k) {
      const int row = min(row0 + (wave * RW + k) * 32 + l32, rows - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(lat + (int64_t)row * R);
#pragma unroll
      for (int s = 0; s < KS; ++s) bl[k][s] = __builtin_bit_cast(bf16x8, src[2 * s + half]);
    }
  }
  // These loads complete here, so no wait for them lands inside the loop (where it would also
  // wait for the stage copies in flight).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // wave-uniform: the wave holds row tiles of this chunk and some of them are real rows
  const bool active = wave * RW < TR && row0 + wave * RW * 32 < rows;

  const uint32_t lds0 = (uint32_t)(uintptr_t)&s_stage[0][0];
  // Per-lane byte offsets of the copies, relative to the step's w2 tile and to the first base row
  // of the copy instruction at the step's first id (loop-invariant; the step only moves the
  // scalar base pointers). A base copy instruction covers 16 rows, and its first row's offset
  // from the chunk (rowb, uniform) is added to the scalar pointer, so a lane offset spans at most
  // 15 rows: 32 bits hold it for any base_ld <= 2^27. In the last step of the vocabulary, ids
  // past V are clamped instead (w2 row V-1, the padded row's last chunk). Copy instruction ins,
  // lane j of the w2 tile carries chunk j % RQ of A-row (j / RQ) * NI + ins.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t offw[WI], offb[BI];
  int64_t rowb[BI];
#pragma unroll
  for (int q = 0; q < WI; ++q) {
    const int ins = (wave + q * kNW) % NI;
    const int i = (lane / RQ) * NI + ins, c = lane % RQ;
    offw[q] = (uint32_t)((w2_row_id(i) * R + 8 * c) * 2);
  }
#pragma unroll
  for (int q = 0; q < BI; ++q) {
    const int ins = (wave_s + q * kNW) % NBI;
    const int r_ins = min(row0 + 16 * ins, rows - 1) - row0;  // the instruction's first row
    rowb[q] = (int64_t)r_ins * ld * 2;
    const int p = ins * 64 + lane;  // base chunk position
    const int rr = p >> 2, c = (p & 3) ^ ((rr >> 2) & 3);
    offb[q] = (uint32_t)(((int64_t)(min(row0 + rr, rows - 1) - row0 - r_ins) * ld + 8 * c) * 2);
  }
  const uint16_t* base_rc = base + (int64_t)row0 * ld;
  // The lane id, recomputed where it is used: the clamped offsets of the vocabulary's last step
  // are needed once per launch, so nothing of them may be hoisted into registers held across the
  // loop.
  auto opaque_lane_id = []() __attribute__((always_inline)) {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  };
  // Issue the copies of step t into stage st. The LDS destinations are scalar (the wave index is
  // uniform), and one uniform branch per step picks the clamped offsets of the vocabulary's last
  // step, so the common path is the copies alone.
  auto copy_step = [&](int t, int st) __attribute__((always_inline)) {
    const uint32_t sbase = lds0 + (uint32_t)st * (SCH * 16);
    const uint16_t* gw = w2 + (int64_t)t * 32 * R;
    const uint16_t* gb = base_rc + 32 * t;
    if (32 * t + 32 > V) {  // uniform: the last step of the vocabulary
#pragma unroll
      for (int q = 0; q < WI; ++q) {
        const int ins = (wave_s + q * kNW) % NI;
        const int ln = opaque_lane_id();
        const int i = (ln / RQ) * NI + ins, c = ln % RQ;
        const uint32_t off = (uint32_t)(((min(32 * t + w2_row_id(i), V - 1) - 32 * t) * R + 8 * c) * 2);
        lds_copy16(gw, off, sbase + ins * WP * 16);
      }
#pragma unroll
      for (int q = 0; q < BI; ++q) {
        const int ins = (wave_s + q * kNW) % NBI;
        const int r_ins = min(row0 + 16 * ins, rows - 1) - row0;
        const int p = ins * 64 + opaque_lane_id();
        const int rr = p >> 2, c = (p & 3) ^ ((rr >> 2) & 3);
        const uint32_t off = (uint32_t)(((int64_t)(min(row0 + rr, rows - 1) - row0 - r_ins) * ld +
                                         8 * (min(4 * t + c, last_chunk) - 4 * t)) * 2);
        lds_copy16(reinterpret_cast<const char*>(gb) + rowb[q], off, sbase + (WCH + ins * 64) * 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < WI; ++q)
        lds_copy16(gw, offw[q], sbase + ((wave_s + q * kNW) % NI) * WP * 16);
#pragma unroll
      for (int q = 0; q < BI; ++q)
        lds_copy16(reinterpret_cast<const char*>(gb) + rowb[q], offb[q],
                   sbase + (WCH + ((wave_s + q * kNW) % NBI) * 64) * 16);
    }
  };

  // this lane's A-fragment chunk of fragment 0 inside a stage (fragment s is 2*s chunks on)
  const int a_off = (l32 % NI) * WP + (l32 / NI) * RQ + half;

  float bv[RW];
  int bi[RW];
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    bv[k] = -INFINITY;
    bi[k] = 32 * t0;
  }
  // Step t of row tile k: the 16 logits of this lane's row (ids 32t + 16*half + e, e = 0..15)
  // folded into the running winner, in three phases. The step maximum comes from a tree of max
  // operations; the lowest e holding it from a descent that takes the upper half at a level only
  // when the lower one lacks the maximum, picking the next level's candidates by multiplexing on
  // the bits found so far. Steps rise with t, so a strict comparison keeps the lowest id among
  // equal values. Only the last step of a range can reach past V (checked when `last` is set).
  struct Epi {
    float m2[8], m4[4], m8[2], sv;  // phase 0 -> 1
    float r1;                       // phase 1 -> 2: the candidate for the last bit
    int se;                         // phase 1 -> 2: the upper three bits of e
  };
  auto epi_phase = [&](int ph, int t, int k, f32x16& acc, Epi& ep, bool last)
      __attribute__((always_inline)) {
    if (ph == 0) {
      if (last && 32 * t + 32 > V) {  // the last step of the vocabulary: ids >= V never win
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * t + 16 * half + e >= V) acc[e] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ep.m2[e] = fmaxf(acc[2 * e], acc[2 * e + 1]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ep.m4[e] = fmaxf(ep.m2[2 * e], ep.m2[2 * e + 1]);
      ep.m8[0] = fmaxf(ep.m4[0], ep.m4[1]);
      ep.m8[1] = fmaxf(ep.m4[2], ep.m4[3]);
      ep.sv = fmaxf(ep.m8[0], ep.m8[1]);
    } else if (ph == 1) {
      const bool c8 = ep.m8[0] != ep.sv;
      const bool c4 = (c8 ? ep.m4[2] : ep.m4[0]) != ep.sv;
      const float q2a = c8 ? ep.m2[4] : ep.m2[0], q2b = c8 ? ep.m2[6] : ep.m2[2];
      const bool c2 = (c4 ? q2b : q2a) != ep.sv;
      float lg[16];  // scalars: a select between two vector elements would become a dynamic index
#pragma unroll
      for (int e = 0; e < 16; ++e) lg[e] = acc[e];
      float q1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q1[j] = c8 ? lg[8 + 2 * j] : lg[2 * j];
      const float r1a = c4 ? q1[2] : q1[0], r1b = c4 ? q1[3] : q1[1];
      ep.r1 = c2 ? r1b : r1a;
      ep.se = (c8 ? 8 : 0) + (c4 ? 4 : 0) + (c2 ? 2 : 0);
    } else {
      ep.se += ep.r1 != ep.sv ? 1 : 0;
      const bool gt = ep.sv > bv[k];
      bv[k] = gt ? ep.sv : bv[k];
      bi[k] = gt ? 32 * t + 16 * half + ep.se : bi[k];
    }
  };
  auto epilogue = [&](int t, int k, f32x16& acc, bool last) __attribute__((always_inline)) {
    Epi ep;
#pragma unroll
    for (int ph = 0; ph < 3; ++ph) epi_phase(ph, t, k, acc, ep, last);
  };

  // The MFMAs of the current stage into acc, with the epilogue of the previous step (tp, accp)
  // when `with_prev` is set: its phases go between the MFMA groups in program order (phase ph of
  // tile k after fragment group 1 + 3*k + ph), so they issue while the matrix core works instead
  // of after it.
  constexpr bool kSpread = 3 * RW + 1 <= KS;
  int st = 0;
  auto compute = [&](f32x16 (&acc)[RW], auto with_prev, int tp, f32x16 (&accp)[RW])
      __attribute__((always_inline)) {
    constexpr bool kPrev = decltype(with_prev)::value != 0;
    const uint4* sp = s_stage[st];
    Epi ep[RW];
    // The accumulators start at the row's base logits: this lane's 16 ids (two 16-byte chunks of
    // the base row) widened from bf16 to fp32 exactly (a shift or a mask per value).
#pragma unroll
    for (int k = 0; k < RW; ++k) {
      const int rr = (wave * RW + k) * 32 + l32;
      const int sw = (rr >> 2) & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 c = sp[WCH + 4 * rr + ((2 * half + h) ^ sw)];
        const uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[k][8 * h + 2 * j] = __uint_as_float(d[j] << 16);
          acc[k][8 * h + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
        }
      }
    }
    // A fragments are read two groups ahead of their MFMAs (three registers sets in rotation).
    const uint4* sa = sp + a_off;
    bf16x8 af[3];
    af[0] = as_bf16x8(sa[0]);
    if constexpr (KS > 1) af[1] = as_bf16x8(sa[2]);
    static_for<0, KS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 2 < KS) af[(s + 2) % 3] = as_bf16x8(sa[2 * (s + 2)]);
#pragma unroll
      for (int k = 0; k < RW; ++k) acc[k] = mfma32x32x16(af[s % 3], bl[k][s], acc[k]);
      if constexpr (kSpread && kPrev && s >= 1 && s <= 3 * RW) {
        constexpr int g = s - 1;
        epi_phase(g % 3, tp, g / 3, accp[g / 3], ep[g / 3], false);
      }
    });
    if constexpr (!kSpread && kPrev) {
#pragma unroll
      for (int k = 0; k < RW; ++k) epilogue(tp, k, accp[k], false);
    }
    // The descent results are consumed here, at the end of the step, so the compiler computes
    // them on every step rather than branching around them where the maximum does not rise (a
    // branch would split the step into separate scheduling regions).
    if constexpr (kSpread && kPrev) {
#pragma unroll
      for (int k = 0; k < RW; ++k) asm volatile("" ::"v"(ep[k].se));
    }
  };
  constexpr int VW = (NS - 2) * DI;  // copies allowed in flight past step t
  // Start step t: this wave's copies of step t are done (those of later steps may still run);
  // after the barrier every wave's are, and every wave has finished reading step t-1's stage,
  // which then receives the copies of step t+NS-1 (past the range end: the last step again, L2
  // hits).
  auto begin_step = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (VW & 15) | ((VW >> 4) << 14));  // vmcnt(VW)
    __syncthreads();
    copy_step(min(t + NS - 1, t1 - 1), st == 0 ? NS - 1 : st - 1);
  };
  auto next_stage = [&]() __attribute__((always_inline)) { st = st == NS - 1 ? 0 : st + 1; };

  // prologue: steps t0 .. t0+NS-2 in flight
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) copy_step(min(t0 + i, t1 - 1), i);
  // Software pipeline: step t's MFMAs carry step t-1's epilogue (VALU, from registers); two
  // accumulator sets alternate. The last epilogue of the range runs on its own.
  f32x16 accA[RW], accB[RW];
  begin_step(t0);
  if (active) compute(accA, Int<0>{}, 0, accB);
  next_stage();
  int t = t0 + 1;
  for (; t + 1 < t1; t += 2) {
    begin_step(t);
    if (active) compute(accB, Int<1>{}, t - 1, accA);
    next_stage();
    begin_step(t + 1);
    if (active) compute(accA, Int<1>{}, t, accB);
    next_stage();
  }
  if (t < t1) {  // one step left: t = t1 - 1
    begin_step(t);
    if (active) {
      compute(accB, Int<1>{}, t - 1, accA);
#pragma unroll
      for (int k = 0; k < RW; ++k) epilogue(t, k, accB[k], true);
    }
  } else if (active) {
#pragma unroll
    for (int k = 0; k < RW; ++k) epilogue(t - 1, k, accA[k], true);
  }
  // drain the trailing copies before the workgroup's LDS can be handed to another workgroup
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // lanes l and l^32 hold the same row with the two halves of each step
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    float v = bv[k];
    int i = bi[k];
    const float ov = __shfl_xor(v, 32);
    const int oi = __shfl_xor(i, 32);
    argmax_merge(v, i, ov, oi);
    const int row = row0 + (wave * RW + k) * 32 + l32;
    // range-major partials: the 32 lanes store 256 contiguous bytes (scattered 8-byte stores
    // into row-major partials cost a partial-line write-back per row at the end of the kernel)
    if (half == 0 && wave * RW < TR && row < rows)
      part[(int64_t)vr * rows + row] = make_uint2(__float_as_uint(v), (unsigned)i);
  }
}

// Partials of RR consecutive rows per workgroup (64, or 16 for a few rows), S = 256/RR range
// slices per row: thread (row lr, slice j) scans ranges j, j+S, ... with up to 16 loads in flight
// (at 64 rows each wave reads 64 consecutive rows of one range: 512 contiguous bytes), the S
// slice winners of a row are merged in LDS, and the row's winner is written into blk in place.
// With passes_run (the last pass of a step, pass = K-1): workgroup 0 also writes the number of
// passes that ran, which flags[0 .. K-2] already fix (pass p >= 1 ran iff pass p-1 changed a
// slot), so the step needs no launch of its own for it.
template <int RR>
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const uint2* __restrict__ part,
                                                            int ntiles, int rows, int B,
                                                            int64_t* __restrict__ blk,
                                                            int32_t* changed, int32_t* flags,
                                                            int pass, int32_t* passes_run) {
  constexpr int S = 256 / RR;
  if (passes_run && blockIdx.x == 0 && threadIdx.x == 0) {
    int n = pass + 1;
    if (flags) {
      n = 1;
      for (int q = 0; q < pass; ++q) n += flags[q] != 0;
    }
    *passes_run = n;
  }
  if (pass_skipped(flags, pass)) return;
  __shared__ float s_v[S][RR];
  __shared__ int s_i[S][RR];
  const int lr = threadIdx.x % RR, j = threadIdx.x / RR;
  const int p = blockIdx.x * RR + lr;
  float bv = -INFINITY;
  int bi = INT_MAX;
  if (p < rows) {
    const uint2* pr = part + p;
    // 16 loads in flight: ranges j + S*(u + 16 i), clamped to the last range (repeats change
    // nothing)
    for (int t0 = j; t0 < ntiles; t0 += 16 * S) {
      uint2 q[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) q[u] = pr[(int64_t)min(t0 + S * u, ntiles - 1) * rows];
#pragma unroll
      for (int u = 0; u < 16; ++u) argmax_merge(bv, bi, __uint_as_float(q[u].x), (int)q[u].y);
    }
  }
  s_v[j][lr] = bv;
  s_i[j][lr] = bi;
  __syncthreads();
  if (j == 0 && p < rows) {
#pragma unroll
    for (int u = 1; u < S; ++u) argmax_merge(bv, bi, s_v[u][lr], s_i[u][lr]);
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

template <int R, int NW, int RW, int NS, int TR>
hipError_t launch_partial_t(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                            int64_t ld, int rows, int64_t V, uint2* part, const int32_t* flags,
                            int pass, hipStream_t s, bool lat_frag) {
  const int nvr = readout_tiles(V, rows);
  constexpr int CH = TR * 32;
  const int n_rc = (rows + CH - 1) / CH;
  hipLaunchKernelGGL((readout_partial_kernel<R, NW, RW, NS, TR>), dim3((unsigned)(nvr * n_rc)), dim3(64 * NW),
                     0, s, lat, w2, base, ld, rows, (int)V, nvr, n_rc, part, flags, pass,
                     lat_frag ? 1 : 0);
  return hipGetLastError();
}

// Row chunk shape: up to 32 rows (a single request), one 32-row tile held by wave 0 while all 8
// waves issue copies, with a base stage of those 32 rows only (a 256-row stage copies the last row
// over and over: 16.2 against 15.2 us at 15 rows; deeper rings, possible with the small stage,
// measured slower: 15.7 us with 4 stages, 17.8 with 8, as the steps in flight outgrow the L2);
// up to 256 rows, 8 waves of one 32-row tile each; more rows, 8 waves of two 32-row tiles each
// (512 rows per chunk), so each w2 fragment read from LDS feeds two MFMAs. (Four waves of four
// tiles, or sixteen of one, measured slower at 480 rows.)
template <int NW, int RW, int NS, int TR = NW * RW>
hipError_t launch_partial_shape(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                                int64_t ld, int rows, int64_t V, int r, uint2* part,
                                const int32_t* flags, int pass, hipStream_t s, bool lat_frag) {
  switch (r) {
    case 64: return launch_partial_t<64, NW, RW, NS, TR>(lat, w2, base, ld, rows, V, part, flags, pass, s, lat_frag);
    case 128: return launch_partial_t<128, NW, RW, NS, TR>(lat, w2, base, ld, rows, V, part, flags, pass, s, lat_frag);
    case 256: return launch_partial_t<256, NW, RW, NS, TR>(lat, w2, base, ld, rows, V, part, flags, pass, s, lat_frag);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Up to 512 rows a launch is one row chunk and the vocabulary is cut into 256 ranges (one
// workgroup per CU); with n_rc > 1 chunks of 512 rows, into about 256 / n_rc ranges (a multiple of
// 8, at least 8), so the launch is still about one workgroup per CU, each over a longer range: the
// lat loads and the copy ring's start are paid once per workgroup (3840 rows: 32 ranges, 357-360
// us against 399-414 us with 256 ranges, 364 with 64, 375 with 128; 48 ranges, 384 workgroups,
// leave half the CUs a second round: 400 us).
int readout_tiles(int64_t V, int rows) {
  const int64_t steps = (V + 31) / 32;
  const int n_rc = rows <= 512 ? 1 : (rows + 511) / 512;
  const int target = n_rc == 1 ? kMaxRanges : max(8, (kMaxRanges / n_rc) & ~7);
  return (int)(steps < target ? steps : target);
}

hipError_t launch_readout_partial(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                                  int64_t ld, int rows, int64_t V, int r, uint2* part,
                                  const int32_t* flags, int pass, hipStream_t s, bool lat_frag) {
  if (rows <= 32) return launch_partial_shape<8, 1, 3, 1>(lat, w2, base, ld, rows, V, r, part, flags, pass, s, lat_frag);
  if (rows <= 256) return launch_partial_shape<8, 1, 3>(lat, w2, base, ld, rows, V, r, part, flags, pass, s, lat_frag);
  return launch_partial_shape<8, 2, 3>(lat, w2, base, ld, rows, V, r, part, flags, pass, s, lat_frag);
}

hipError_t launch_argmax_reduce(const uint2* part, int ntiles, int rows, int B, int64_t* blk,
                                int32_t* changed, int32_t* flags, int pass, hipStream_t s,
                                int32_t* passes_run) {
  if (rows <= 16)
    hipLaunchKernelGGL(argmax_reduce_kernel<16>, dim3(1), dim3(256), 0, s, part, ntiles, rows, B,
                       blk, changed, flags, pass, passes_run);
  else
    hipLaunchKernelGGL(argmax_reduce_kernel<64>, dim3((rows + 63) / 64), dim3(256), 0, s, part,
                       ntiles, rows, B, blk, changed, flags, pass, passes_run);
  return hipGetLastError();
}

}  // namespace xpress
