// Shared device helpers of the XPress pass kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace xpress {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (inputs finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// (value, index) arg-max combine: larger value wins; equal values keep the lower index.
// -0.0 and +0.0 compare equal, so they tie and the lower index wins.
// Compile-time loop: f(Int<i>{}) for i = I .. N-1, each body instantiated with a constant index
// (a plain unrolled loop is not guaranteed to unroll once its body grows, and a rolled loop
// indexes register arrays dynamically).
template <int V> struct Int { static constexpr int value = V; };
template <int I, int N, class F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  const bool take = (ov > v) | ((ov == v) & (oi < i));  // bitwise: no branches
  v = take ? ov : v;
  i = take ? oi : i;
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads of 16 and 8 bytes: data read once per pass.
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Element offset of lat[p, c] (readout row p, channel c) in the fragment order that a step's
// full-vocabulary readout loads with one contiguous 1 KiB read per wave instruction: row tile
// T = p / 32 holds, for each 16-channel k-step s and lane l = 32*half + p%32, the 8 channels
// 16s + 8*half .. +7 of row p as one 16-byte chunk at chunk index (T*(R/16) + s)*64 + l -- the
// B-operand fragment of v_mfma_f32_32x32x16_bf16 that lane l holds for k-step s. A buffer of
// ceil(rows/32) whole tiles holds it.
template <int R>
__device__ __forceinline__ int64_t lat_frag_offset(int p, int c) {
  const int T = p >> 5, lr = p & 31, q = c >> 3;
  return ((int64_t)(T * (R / 16) + (q >> 1)) * 64 + (q & 1) * 32 + lr) * 8 + (c & 7);
}

// One 1 KiB copy from global memory straight into LDS (global_load_lds_dwordx4: no registers):
// this lane's 16 bytes at gbase + off (a scalar base pointer and a per-lane 32-bit byte offset)
// to LDS byte address lds_base + 16 * lane. Written as inline assembly so the compiler's
// wait-count bookkeeping stays out of it: the caller waits for the copies itself, with vmcnt,
// before the barrier that publishes them.
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t off, uint32_t lds_base) {
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(off), "s"(gbase) : "memory");
}

// Skip test of the fixed-point early exit: pass p >= 1 is skipped once pass p-1 changed nothing.
// flags == nullptr disables it.
__device__ __forceinline__ bool pass_skipped(const int32_t* flags, int pass) {
  return flags != nullptr && pass > 0 && flags[pass - 1] == 0;
}

}  // namespace xpress
