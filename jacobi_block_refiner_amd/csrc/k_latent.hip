// Latent stage of one XPress pass (gfx950): two kernels from a projected embedding table, or
// three wide kernels that project the gathered embeddings themselves.
//
// For every block (vLLM API page "vllm.v1.worker.gpu.spec_decode.xpress.kernels",
// _xpress_latent_kernel docstring; "vllm.model_executor.models.qwen3_xpress",
// XPressRefinerHead._refine_latent):
//   1. gather the embedding of each slot's previous token: slot 0 reads am1, slot b reads blk[b-1];
//   2. x = xh + P_e . e with P_e = in_proj[:, 2r:3r];
//   3. per-channel causal mixer u[b, c] = sum_{j<=b} L[b, j, c] x[j, c] (L stored [B, B, r]);
//   4. SwiGLU: s = silu(w_gate . u) * (w_up . u);
//   5. lat = u + w_down . s for slots 1..B-1 (slot 0 is never read out).
// A block's 16 slots (padded with zero rows past B) are the M = 16 rows of a
// v_mfma_f32_16x16x32_bf16 tile. One workgroup per block cannot keep enough CUs busy at small N
// (each block-pass needs ~1 MB of weights, which one CU pulls from L2 in several microseconds), so
// the stage is split where a full reduction over channels is needed:
//   latent_mix_kernel   (block, 64-channel slice): steps 1-3, u in fp32 and bf16 to scratch
//                       (inside a step it also finishes the previous pass's argmax);
//   latent_gate_kernel  (row tile, 64 hidden units): step 4, s in bf16 to scratch;
//   latent_down_kernel  (row tile, 64 channels): step 5, lat in bf16.
// Each workgroup reads at most 64 KB of weights; row tiles of 64 rows (4 blocks) share weight
// reads when there are many blocks.
// With the projected table w1p = P_e applied to every row of w1 (fold_embedding_kernel, once per
// weight set), step 2 is a row gather, and while N * M/64 <= 448 the stage runs as
//   latent_share_kernel (block, 64 hidden units): steps 1-4 and the slice's share of step 5;
//   latent_sum_kernel   (block, slots): the shares summed in slice order into lat.
//
// v_mfma_f32_16x16x32_bf16 operand layout (wave64):
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) + e, e = 0..7
//   B (32 x 16): lane l holds col l%16, the same k
//   D (16 x 16): lane l, accumulator v holds row 4*(l/16) + v, col l%16
#include "launch.hpp"
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

namespace {

// block_tokens_*: the token each of the 16 slots of block n reads (slot 0: am1[n], slot b:
// blk[n, b-1]; -1 for slots past B) into tok (LDS). With `part` (inside a step, pass >= 1) the
// block first finishes the previous pass: the partial winners of its readout rows (range-major,
// `ntiles` <= 256 ranges) are reduced to the block's new tokens -- the work of the argmax-reduce
// kernel for these rows, without its launch. Every workgroup of the block reduces them (the same
// result); the one with `writer` set writes them into blk and raises flags[pass-1] on a change.
// Two halves, so that a kernel can issue the partials' loads (the head of its dependency chain)
// before its other loads and reduce them after: block_tokens_load fills this thread's 16
// partials (lane l of wave w: readout row l%16 of the block, ranges 4*(16w + k) + l/16, so one
// load instruction of a wave reads four ranges' contiguous rows of the block; clamped repeats
// change nothing), block_tokens_finish reduces them (q is ignored without part). Both are called
// by all 256 threads; the caller synchronises before reading tok.
__device__ __forceinline__ void block_tokens_load(const uint2* __restrict__ part, int ntiles,
                                                  int rows, int n, int B, uint2 (&q)[16]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rb = lane & 15, sub = lane >> 4;
  const uint2* pr = part + (int64_t)n * (B - 1) + min(rb, B - 2);
#pragma unroll
  for (int k = 0; k < 16; ++k) q[k] = pr[(int64_t)min((w * 16 + k) * 4 + sub, ntiles - 1) * rows];
}

__device__ __forceinline__ void block_tokens_finish(bool has_part, const uint2 (&q)[16],
                                                    int64_t* __restrict__ blk,
                                                    const int64_t* __restrict__ am1, int n, int B,
                                                    bool writer, int32_t* __restrict__ flags,
                                                    int pass, int64_t* tok) {
  const int tid = threadIdx.x;
  if (has_part) {
    __shared__ float s_bv[4][16];
    __shared__ int s_bi[4][16];
    const int lane = tid & 63, w = tid >> 6, rb = lane & 15;  // readout row rb of the block
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (rb < B - 1) {
#pragma unroll
      for (int k = 0; k < 16; ++k) argmax_merge(bv, bi, __uint_as_float(q[k].x), (int)q[k].y);
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {  // the wave's four lanes of row rb
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      argmax_merge(bv, bi, ov, oi);
    }
    if (lane < 16) {
      s_bv[w][lane] = bv;
      s_bi[w][lane] = bi;
    }
    __syncthreads();
    if (tid < B - 1) {  // the four waves' winners of row tid
      bv = s_bv[0][tid];
      bi = s_bi[0][tid];
#pragma unroll
      for (int k = 1; k < 4; ++k) argmax_merge(bv, bi, s_bv[k][tid], s_bi[k][tid]);
      const int64_t nv = (int64_t)bi;
      if (writer) {
        int64_t* slot = blk + (int64_t)n * B + 1 + tid;
        if (*slot != nv) {
          *slot = nv;
          if (flags) __hip_atomic_store(flags + pass - 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (tid + 2 < B) tok[tid + 2] = nv;  // slot b reads blk[b-1]
    }
    if (tid == 0) {
      tok[0] = am1[n];
      tok[1] = blk[(int64_t)n * B];
    }
    if (tid >= B && tid < 16) tok[tid] = -1;
  } else if (tid < 16) {
    tok[tid] = tid == 0 ? am1[n] : (tid < B ? blk[(int64_t)n * B + tid - 1] : -1);
  }
}

// The mixer rows of wave w in latent_mix_kernel: w, 15-w, w+4 and 11-w, two pairs (b, 15-b) of
// 17 taps each (row b has the b+1 taps j <= b), so every wave loads and multiplies 34 taps per
// channel.
constexpr int mix_row(int w, int k) { return k == 0 ? w : k == 1 ? 15 - w : k == 2 ? w + 4 : 11 - w; }
constexpr int mix_tap0(int w, int k) { return k == 0 ? 0 : mix_tap0(w, k - 1) + mix_row(w, k - 1) + 1; }

// Steps 1-3 for one block and 64 channels (blockIdx.y); 4 waves. With `part` given (inside a
// step), the block first finishes the previous pass (block_tokens_*); slice 0 writes blk.
template <int R>
__global__ __launch_bounds__(256) void latent_mix_kernel(
    const uint2* __restrict__ part, int ntiles, int rows, int64_t* __restrict__ blk,
    const int64_t* __restrict__ am1, const float* __restrict__ xh, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ in_proj, const uint16_t* __restrict__ mix_L, int B, int64_t V,
    float* __restrict__ u32, uint16_t* __restrict__ u16, int32_t* __restrict__ flags, int pass) {
  // fused: runs when the previous pass ran; plain: when this pass runs
  if (part ? pass_skipped(flags, pass - 1) : pass_skipped(flags, pass)) return;
  constexpr int EP = R + 8;  // bf16 row pitch of s_e (a 16-byte pad per row)
  __shared__ int64_t s_tok[16];
  __shared__ float s_x[16][65];
  __shared__ __align__(16) uint16_t s_e[16][EP];
  const int n = blockIdx.x, c0 = blockIdx.y * 64, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, q4 = lane >> 4;

  // The previous pass's partials first (they head the dependency chain), then the mixer taps of
  // this thread's channel c0 + lane for the wave's rows (mix_row; independent of the tokens):
  // mix_L is [B, B, r], channel innermost, so a tap is one coalesced 2-byte load across the wave.
  // Rows past B are zeroed after the mixer. The wave index is uniform, so each wave runs its own
  // copy of the tap loads and the mixer, with every index known at compile time.
  uint2 qp[16];
  if (part) block_tokens_load(part, ntiles, rows, n, B, qp);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint16_t tap[34];
  auto load_taps = [&](auto wc) __attribute__((always_inline)) {
    constexpr int W = decltype(wc)::value;
    static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value, b = mix_row(W, K), e0 = mix_tap0(W, K);
      static_for<0, b + 1>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        tap[e0 + j] = mix_L[(int64_t)(min(b, B - 1) * B + min(j, B - 1)) * R + c0 + lane];
      });
    });
  };
  static_for<0, 4>([&](auto wc) __attribute__((always_inline)) {
    if (wave_s == decltype(wc)::value) load_taps(wc);
  });

  block_tokens_finish(part != nullptr, qp, blk, am1, n, B, blockIdx.y == 0, flags, pass, s_tok);
  __syncthreads();

  // steps 1-2: x[slot, c] = xh[slot, c] + sum_k P_e[c, k] w1[tok(slot), k]; wave w computes the
  // 16 x 16 tile of channels c0 + 16w .. +15 (A: the 16 slots' embeddings, B: P_e rows). The 16
  // embedding rows are read once per workgroup into LDS (every wave multiplies all of them).
  {
    constexpr int RC = R / 8, NCH = 16 * RC, PER = (NCH + 255) / 256;
    uint4 ev[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = min(tid + 256 * i, NCH - 1), slot = idx / RC;
      const int64_t tok = slot < B ? s_tok[slot] : -1;
      const bool live = tok >= 0 && tok < V;  // slots past B and ids outside [0, V): zero
      ev[i] = *reinterpret_cast<const uint4*>(w1 + (live ? tok : 0) * R + 8 * (idx % RC));
      if (!live) ev[i] = make_uint4(0, 0, 0, 0);
    }
    const int c = c0 + 16 * wave + l16;
    const uint4* prow = reinterpret_cast<const uint4*>(in_proj + (int64_t)c * 3 * R + 2 * R);
    bf16x8 a[R / 32], b[R / 32];
#pragma unroll
    for (int s2 = 0; s2 < R / 32; ++s2) b[s2] = as_bf16x8(prow[4 * s2 + q4]);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i;
      if (idx < NCH) *reinterpret_cast<uint4*>(&s_e[idx / RC][8 * (idx % RC)]) = ev[i];
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < R / 32; ++s2)
      a[s2] = as_bf16x8(*reinterpret_cast<const uint4*>(&s_e[l16][32 * s2 + 8 * q4]));
    float h[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int slot = 4 * q4 + v;
      h[v] = slot < B ? xh[((int64_t)n * B + slot) * R + c] : 0.f;
    }
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s2 = 0; s2 < R / 32; ++s2) acc = mfma16x16x32(a[s2], b[s2], acc);
#pragma unroll
    for (int v = 0; v < 4; ++v) s_x[4 * q4 + v][16 * wave + l16] = acc[v] + h[v];
  }
  __syncthreads();

  // step 3: u[b, c] = sum_{j<=b} L[b, j, c] x[j, c]; thread -> channel c0 + lane, the wave's
  // rows mix_row(wave, 0..3)
  {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = s_x[j][lane];
    float* o32 = u32 + (int64_t)n * 16 * R + c0 + lane;
    uint16_t* o16 = u16 + (int64_t)n * 16 * R + c0 + lane;
    auto mix = [&](auto wc) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value, b = mix_row(W, K), e0 = mix_tap0(W, K);
        float u = 0.f;
        static_for<0, b + 1>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          u = fmaf(bf16_to_f32(tap[e0 + j]), x[j], u);
        });
        u = b < B ? u : 0.f;
        o32[(int64_t)b * R] = u;
        o16[(int64_t)b * R] = f32_to_bf16(u);
      });
    };
    static_for<0, 4>([&](auto wc) __attribute__((always_inline)) {
      if (wave_s == decltype(wc)::value) mix(wc);
    });
  }
}

// Rows r0 .. r0+nr-1 of a bf16 matrix with `ld` elements per row, columns k0 .. k0+KW-1, copied
// into LDS rows of pitch P elements (a 16-byte pad per row keeps the 16 rows of an MFMA fragment
// read on distinct banks). Rows past nrows repeat the last one (their results are not stored).
// Called by all 256 threads; the caller synchronises before reading.
template <int NR, int KW, int P>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int64_t ld, int r0,
                                           int nrows, int k0, uint16_t (*dst)[P]) {
  constexpr int RC = KW / 8;        // 16-byte chunks per row
  constexpr int NCH = NR * RC;
  constexpr int PER = (NCH + 255) / 256;
  uint4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // all loads before any store
    const int idx = min((int)threadIdx.x + 256 * i, NCH - 1);
    const int r = min(r0 + idx / RC, nrows - 1);
    v[i] = *reinterpret_cast<const uint4*>(src + (int64_t)r * ld + k0 + 8 * (idx % RC));
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = (int)threadIdx.x + 256 * i;
    if (idx < NCH) *reinterpret_cast<uint4*>(&dst[idx / RC][8 * (idx % RC)]) = v[i];
  }
}

// Step 4 for rows r0..r0+16*G-1 (whole blocks, 16 rows each) and hidden units h0..h0+63; wave w
// owns units h0 + 16w .. +15. The rows of u are read once per workgroup into LDS (every wave
// multiplies all of them) and each wave keeps its own units' gate and up rows in registers.
template <int R, int G>
__global__ __launch_bounds__(256) void latent_gate_kernel(
    const uint16_t* __restrict__ u16, const uint16_t* __restrict__ w_gate,
    const uint16_t* __restrict__ w_up, int M, int nrows, uint16_t* __restrict__ s16,
    const int32_t* __restrict__ flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int AP = R + 8;
  __shared__ __align__(16) uint16_t s_a[16 * G][AP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int r0 = blockIdx.x * 16 * G;
  const int m = blockIdx.y * 64 + wave * 16 + l16;
  const uint4* grow = reinterpret_cast<const uint4*>(w_gate + (int64_t)m * R);
  const uint4* urow = reinterpret_cast<const uint4*>(w_up + (int64_t)m * R);
  f32x4 ag[G], au[G];
#pragma unroll
  for (int g = 0; g < G; ++g) ag[g] = au[g] = f32x4{0, 0, 0, 0};
  // all operands are loaded before the first MFMA, so their latencies overlap
  bf16x8 bg[R / 32], bu[R / 32];
#pragma unroll
  for (int s = 0; s < R / 32; ++s) {
    bg[s] = as_bf16x8(grow[4 * s + q4]);
    bu[s] = as_bf16x8(urow[4 * s + q4]);
  }
  stage_rows<16 * G, R, AP>(u16, R, r0, nrows, 0, s_a);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < R / 32; ++s)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&s_a[16 * g + l16][32 * s + 8 * q4]));
      ag[g] = mfma16x16x32(a, bg[s], ag[g]);
      au[g] = mfma16x16x32(a, bu[s], au[g]);
    }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * g + 4 * q4 + v;
      if (r < nrows) {
        const float x = ag[g][v];
        const float sg = x / (1.f + __expf(-x));
        s16[(int64_t)r * M + m] = f32_to_bf16(sg * au[g][v]);
      }
    }
}

// Step 5 for rows r0..r0+16*G-1 and channels c0..c0+63; wave w owns channels c0 + 16w .. +15.
// The k range (the M hidden units) goes in chunks of 256: the chunk's rows of s are read once per
// workgroup into LDS, while each wave's w_down rows for the chunk are in registers.
template <int R, int G>
__global__ __launch_bounds__(256) void latent_down_kernel(
    const uint16_t* __restrict__ s16, const float* __restrict__ u32,
    const uint16_t* __restrict__ w_down, int M, int B, int nrows, uint16_t* __restrict__ lat,
    const int32_t* __restrict__ flags, int pass, int lat_frag) {
  if (pass_skipped(flags, pass)) return;
  constexpr int KW = 256;           // hidden units per chunk (M is 64 .. 1024, a power of two)
  constexpr int AP = KW + 8;
  __shared__ __align__(16) uint16_t s_a[16 * G][AP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int r0 = blockIdx.x * 16 * G;
  const int c = blockIdx.y * 64 + wave * 16 + l16;
  const uint4* drow = reinterpret_cast<const uint4*>(w_down + (int64_t)c * M);
  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0, 0, 0, 0};
  for (int k0 = 0; k0 < M; k0 += KW) {
    // this chunk's k steps (M = 64 or 128: one partial chunk); indexes past M are clamped and
    // their MFMAs skipped
    const int ns = min(KW, M - k0) / 32;
    bf16x8 b[KW / 32];
#pragma unroll
    for (int i = 0; i < KW / 32; ++i) b[i] = as_bf16x8(drow[(k0 >> 3) + 4 * min(i, ns - 1) + q4]);
    if (k0 > 0) __syncthreads();  // the previous chunk's fragments have been read
    if (M - k0 >= KW) {
      stage_rows<16 * G, KW, AP>(s16, M, r0, nrows, k0, s_a);
    } else {
      // M = 64 or 128: the whole k range is narrower than a chunk
      if (M - k0 == 128) stage_rows<16 * G, 128, AP>(s16, M, r0, nrows, k0, s_a);
      else stage_rows<16 * G, 64, AP>(s16, M, r0, nrows, k0, s_a);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KW / 32; ++i)
      if (i < ns)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&s_a[16 * g + l16][32 * i + 8 * q4]));
          acc[g] = mfma16x16x32(a, b[i], acc[g]);
        }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + 16 * g + 4 * q4 + v;  // row = 16 * block + slot
      const int n = r >> 4, slot = r & 15;
      if (r < nrows && slot >= 1 && slot < B) {
        const int p = n * (B - 1) + slot - 1;
        lat[lat_frag ? lat_frag_offset<R>(p, c) : (int64_t)p * R + c] =
            f32_to_bf16(u32[(int64_t)r * R + c] + acc[g][v]);
      }
    }
}

// Embedding table with the embedding block of in_proj applied (done once per weight set; the
// pass then gathers rows instead of projecting them):
//   w1p[v, c] = sum_k in_proj[c, 2r + k] * w1[v, k]    (fp32)
// Each wave computes 64 vocabulary rows (four 16-row MFMA tiles sharing every in_proj fragment)
// for all r channels.
template <int R>
__global__ __launch_bounds__(256) void fold_embedding_kernel(const uint16_t* __restrict__ w1,
                                                             const uint16_t* __restrict__ in_proj,
                                                             int64_t V, float* __restrict__ w1p) {
  constexpr int KS = R / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int64_t v0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (v0 >= V) return;  // wave-uniform; the kernel has no barrier
  bf16x8 a[4][KS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t row = min(v0 + 16 * t + l16, V - 1);
    const uint4* src = reinterpret_cast<const uint4*>(w1 + row * R);
#pragma unroll
    for (int s = 0; s < KS; ++s) a[t][s] = as_bf16x8(src[4 * s + q4]);
  }
  for (int ct = 0; ct < R / 16; ++ct) {
    const int c = ct * 16 + l16;
    const uint4* prow = reinterpret_cast<const uint4*>(in_proj + (int64_t)c * 3 * R + 2 * R);
    bf16x8 b[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) b[s] = as_bf16x8(prow[4 * s + q4]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma16x16x32(a[t][s], b[s], acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = v0 + 16 * t + 4 * q4 + v;
        if (row < V) w1p[row * R + c] = acc[v];
      }
    }
  }
}

// The latent stage from the projected embedding table w1p, in two launches. Workgroup (n, g)
// of latent_share_kernel takes block n and the 64 SwiGLU units g*64 .. g*64+63 (G = M/64
// workgroups per block):
//   0. the block's tokens (block_tokens_*; inside a step this finishes the previous pass);
//   1. x[b, c] = xh[b, c] + w1p[tok(b), c]            16-byte rows into LDS;
//   2. u[b, c] = sum_{j<=b} L[b, j, c] x[j, c]          lane l: channels CL*l .. +CL-1 (CL = r/64)
//                                                       of the wave's rows mix_row(wave, 0..3);
//   3. a = w_gate[units] . u, e = w_up[units] . u,  s = silu(a) * e   (16x16x32 MFMAs);
//   4. share_g = w_down[:, units] . s (+ u for g = 0), written to dpart for slots 1..B-1.
// latent_sum_kernel then adds the G shares of each slot in slice order into lat (bf16): a fixed
// summation order, and the kernel boundary orders the shares' stores before their loads.
// Every workgroup of a block computes the same u (same inputs, same arithmetic). A slice is UPW
// = 64 units (waves 0-3 take 16 each) or, with few blocks, 32 (waves 0-1; twice the workgroups,
// each with half the gate, up and down weights to load).
template <int R, int UPW>
__global__ __launch_bounds__(256) void latent_share_kernel(
    const uint2* __restrict__ part, int ntiles, int rows, int64_t* __restrict__ blk,
    const int64_t* __restrict__ am1, const float* __restrict__ xh, const float* __restrict__ w1p,
    const uint16_t* __restrict__ mix_L, const uint16_t* __restrict__ w_gate,
    const uint16_t* __restrict__ w_up, const uint16_t* __restrict__ w_down, int B, int M,
    int64_t V, float* __restrict__ dpart, int32_t* __restrict__ flags, int pass) {
  // inside a step: runs when the previous pass ran; on its own: when this pass runs
  if (part ? pass_skipped(flags, pass - 1) : pass_skipped(flags, pass)) return;
  constexpr int KS = R / 32;  // k steps of the gate/up products
  constexpr int DT = R / 64;  // 16-channel output tiles of the down product per wave
  constexpr int UP = R + 8;   // bf16 row pitch of s_u (one 16-byte pad per row)
  constexpr int SP = UPW + 8;  // bf16 row pitch of s_s
  constexpr int UW = UPW / 16;  // waves with units
  constexpr int DK = UPW / 32;  // k steps of the down product
  constexpr int CL = R / 64;    // mixer channels per lane
  constexpr int CW = (CL + 1) / 2;  // 32-bit words of a lane's CL taps
  constexpr int QR = R / 4;     // float4 per x row
  constexpr int NXI = 16 * QR / 256;  // float4 of the x tile per thread
  __shared__ int64_t s_tok[16];
  __shared__ __align__(16) float s_x[16][R];
  __shared__ __align__(16) float s_u32[16][R];
  __shared__ __align__(16) uint16_t s_u[16][UP];
  __shared__ __align__(16) uint16_t s_s[16][SP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int n = blockIdx.x, g = blockIdx.y, G = gridDim.y;

  // The previous pass's partials head the dependency chain (partials -> tokens -> w1p rows), so
  // their loads are issued first (1% faster steps than issuing them after the others); then the
  // loads that do not depend on the tokens: the slice's gate/up rows, xh and the taps.
  uint2 qp[16];
  if (part) block_tokens_load(part, ntiles, rows, n, B, qp);
  const int m = g * UPW + min(wave, UW - 1) * 16 + l16;
  bf16x8 gB[KS], uB[KS];
  if (wave < UW) {  // uniform
    const uint4* grow = reinterpret_cast<const uint4*>(w_gate + (int64_t)m * R);
    const uint4* urow = reinterpret_cast<const uint4*>(w_up + (int64_t)m * R);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      gB[s] = as_bf16x8(grow[4 * s + q4]);
      uB[s] = as_bf16x8(urow[4 * s + q4]);
    }
  }
  // Every load below is unconditional, at an index clamped into range, and a select drops what
  // is not wanted: a load under a condition becomes a branch with its own wait, one memory
  // round trip at a time. xh: thread tid takes the float4 tid + 256 i of the [16, r] x tile.
  float4 xv[NXI];
#pragma unroll
  for (int i = 0; i < NXI; ++i) {
    const int idx = tid + 256 * i, b = idx / QR;
    xv[i] = *reinterpret_cast<const float4*>(xh + ((int64_t)n * B + min(b, B - 1)) * R + 4 * (idx % QR));
  }
  // taps L[b, j, c] of the lane's CL channels for the wave's rows mix_row(wave, 0..3), j <= b
  // (mix_L is [B, B, r], channel innermost: one coalesced 2*CL-byte load per tap across the
  // wave). The wave index is uniform, so each wave runs its own copy of the loads and of the
  // mixer, with every index known at compile time. Rows b >= B are zeroed after the mixer.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t tap[34][CW];
  auto load_taps = [&](auto wc) __attribute__((always_inline)) {
    constexpr int W = decltype(wc)::value;
    static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
      constexpr int K = decltype(kc)::value, b = mix_row(W, K), e0 = mix_tap0(W, K);
      static_for<0, b + 1>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        const uint16_t* t = mix_L + (int64_t)(min(b, B - 1) * B + min(j, B - 1)) * R + CL * lane;
        if constexpr (CL == 4) {
          const uint2 v = *reinterpret_cast<const uint2*>(t);
          tap[e0 + j][0] = v.x;
          tap[e0 + j][1] = v.y;
        } else if constexpr (CL == 2) {
          tap[e0 + j][0] = *reinterpret_cast<const uint32_t*>(t);
        } else {
          tap[e0 + j][0] = *t;
        }
      });
    });
  };
  static_for<0, 4>([&](auto wc) __attribute__((always_inline)) {
    if (wave_s == decltype(wc)::value) load_taps(wc);
  });

  block_tokens_finish(part != nullptr, qp, blk, am1, n, B, g == 0, flags, pass, s_tok);
  __syncthreads();

  // step 1: the x tile into LDS
  {
    float4 e[NXI];
    bool ok[NXI];
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int idx = tid + 256 * i, b = idx / QR;
      const int64_t t = s_tok[b];
      ok[i] = b < B && t >= 0 && t < V;  // slots past B and ids outside [0, V): zero
      e[i] = *reinterpret_cast<const float4*>(w1p + (ok[i] ? t : 0) * R + 4 * (idx % QR));
    }
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int idx = tid + 256 * i, b = idx / QR;
      const bool live = b < B;
      float4 x;
      x.x = live ? xv[i].x + (ok[i] ? e[i].x : 0.f) : 0.f;
      x.y = live ? xv[i].y + (ok[i] ? e[i].y : 0.f) : 0.f;
      x.z = live ? xv[i].z + (ok[i] ? e[i].z : 0.f) : 0.f;
      x.w = live ? xv[i].w + (ok[i] ? e[i].w : 0.f) : 0.f;
      *reinterpret_cast<float4*>(&s_x[b][4 * (idx % QR)]) = x;
    }
  }
  __syncthreads();
  // step 2: the mixer rows of the wave, lane channels CL*lane .. +CL-1
  {
    float x[16][CL];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (CL == 4) {
        const float4 v = *reinterpret_cast<const float4*>(&s_x[j][4 * lane]);
        x[j][0] = v.x; x[j][1] = v.y; x[j][2] = v.z; x[j][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < CL; ++e) x[j][e] = s_x[j][CL * lane + e];
      }
    }
    auto mix = [&](auto wc) __attribute__((always_inline)) {
      constexpr int W = decltype(wc)::value;
      static_for<0, 4>([&](auto kc) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value, b = mix_row(W, K), e0 = mix_tap0(W, K);
        float u[CL];
#pragma unroll
        for (int e = 0; e < CL; ++e) u[e] = 0.f;
        static_for<0, b + 1>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
#pragma unroll
          for (int e = 0; e < CL; ++e) {
            const uint32_t w = tap[e0 + j][e / 2];
            const float l = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            u[e] = fmaf(l, x[j][e], u[e]);
          }
        });
#pragma unroll
        for (int e = 0; e < CL; ++e) {
          u[e] = b < B ? u[e] : 0.f;
          s_u32[b][CL * lane + e] = u[e];
          s_u[b][CL * lane + e] = f32_to_bf16(u[e]);
        }
      });
    };
    static_for<0, 4>([&](auto wc) __attribute__((always_inline)) {
      if (wave_s == decltype(wc)::value) mix(wc);
    });
  }
  // the slice's w_down columns, needed after the gate products
  bf16x8 dB[DT][DK];
#pragma unroll
  for (int it = 0; it < DT; ++it) {
    const int i = (wave * DT + it) * 16 + l16;
    const uint4* drow = reinterpret_cast<const uint4*>(w_down + (int64_t)i * M + g * UPW);
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) dB[it][ks] = as_bf16x8(drow[4 * ks + q4]);
  }
  __syncthreads();

  // step 3: units g*UPW + 16*wave .. +15 for the 16 slot rows
  if (wave < UW) {  // uniform
    f32x4 ag = {0, 0, 0, 0}, au = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&s_u[l16][32 * s + 8 * q4]));
      ag = mfma16x16x32(a, gB[s], ag);
      au = mfma16x16x32(a, uB[s], au);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float z = ag[v];
      const float sg = z / (1.f + __expf(-z));
      s_s[4 * q4 + v][16 * wave + l16] = f32_to_bf16(sg * au[v]);
    }
  }
  __syncthreads();

  // step 4: this slice's share of w_down . s for channels (wave*DT + it)*16 + l16; slice 0's
  // share carries the residual u
  {
    bf16x8 a[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      a[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&s_s[l16][32 * ks + 8 * q4]));
    float* dp = dpart + ((int64_t)n * G + g) * 16 * R;
#pragma unroll
    for (int it = 0; it < DT; ++it) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) acc = mfma16x16x32(a[ks], dB[it][ks], acc);
      const int i = (wave * DT + it) * 16 + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int b = 4 * q4 + v;
        if (b >= 1 && b < B) dp[b * R + i] = g == 0 ? s_u32[b][i] + acc[v] : acc[v];
      }
    }
  }
}

// lat[n, b-1, c] = sum_g dpart[n, g, b, c] in slice order, for slots 1..B-1. Workgroup (n, y)
// takes 256/(r/4) consecutive slots, one thread per 4 channels of a slot; KB shares in flight at
// once (16 when there are more than 8 slices, so that 16 slices take one round trip).
template <int R, int KB>
__global__ __launch_bounds__(256) void latent_sum_kernel(const float* __restrict__ dpart, int B,
                                                         int G, uint16_t* __restrict__ lat,
                                                         const int32_t* __restrict__ flags,
                                                         int pass, int prev, int lat_frag) {
  if (prev ? pass_skipped(flags, pass - 1) : pass_skipped(flags, pass)) return;
  constexpr int QR = R / 4;
  constexpr int RPW = 256 / QR;
  const int n = blockIdx.x, tid = threadIdx.x;
  const int b = 1 + blockIdx.y * RPW + tid / QR, q = tid % QR;
  if (b >= B) return;
  const float4* dp4 = reinterpret_cast<const float4*>(dpart + (int64_t)n * G * 16 * R);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g0 = 0; g0 < G; g0 += KB) {
    // KB shares in flight at once (indexes past G clamped, their values dropped)
    float4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) v[k] = dp4[((int64_t)min(g0 + k, G - 1) * 16 + b) * QR + q];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const bool on = g0 + k < G;
      acc.x += on ? v[k].x : 0.f;
      acc.y += on ? v[k].y : 0.f;
      acc.z += on ? v[k].z : 0.f;
      acc.w += on ? v[k].w : 0.f;
    }
  }
  uint2 o;
  o.x = pack_bf16x2(acc.x, acc.y);
  o.y = pack_bf16x2(acc.z, acc.w);
  const int p = n * (B - 1) + b - 1;
  *reinterpret_cast<uint2*>(lat + (lat_frag ? lat_frag_offset<R>(p, 4 * q) : (int64_t)p * R + 4 * q)) = o;
}

template <int R>
hipError_t launch_r(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                    const float* xh, const uint16_t* w1, const uint16_t* in_proj,
                    const uint16_t* mix_L, const uint16_t* w_gate, const uint16_t* w_up,
                    const uint16_t* w_down, int N, int B, int M, int64_t V, uint16_t* lat,
                    void* scratch, int32_t* flags, int pass, hipStream_t s, bool lat_frag) {
  const int nrows = N * 16;
  const int lf = lat_frag ? 1 : 0;
  float* u32 = static_cast<float*>(scratch);
  uint16_t* u16 = reinterpret_cast<uint16_t*>(u32 + (size_t)nrows * R);
  uint16_t* s16 = u16 + (size_t)nrows * R;
  hipLaunchKernelGGL(latent_mix_kernel<R>, dim3(N, R / 64), dim3(256), 0, s, part, ntiles, N * (B - 1),
                     blk, am1, xh, w1, in_proj, mix_L, B, V, u32, u16, flags, pass);
  const bool wide = N >= 128;  // 4 blocks per workgroup: weights read once per 64 rows
  const int G = wide ? 4 : 1;
  dim3 g2((nrows + 16 * G - 1) / (16 * G), M / 64), g3((nrows + 16 * G - 1) / (16 * G), R / 64);
  if (wide) {
    hipLaunchKernelGGL((latent_gate_kernel<R, 4>), g2, dim3(256), 0, s, u16, w_gate, w_up, M,
                       nrows, s16, flags, pass);
    hipLaunchKernelGGL((latent_down_kernel<R, 4>), g3, dim3(256), 0, s, s16, u32, w_down, M, B,
                       nrows, lat, flags, pass, lf);
  } else {
    hipLaunchKernelGGL((latent_gate_kernel<R, 1>), g2, dim3(256), 0, s, u16, w_gate, w_up, M,
                       nrows, s16, flags, pass);
    hipLaunchKernelGGL((latent_down_kernel<R, 1>), g3, dim3(256), 0, s, s16, u32, w_down, M, B,
                       nrows, lat, flags, pass, lf);
  }
  return hipGetLastError();
}

template <int R>
hipError_t launch_fused_r(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                          const float* xh, const float* w1p, const uint16_t* mix_L,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          int N, int B, int M, int64_t V, uint16_t* lat, float* dpart,
                          int32_t* flags, int pass, hipStream_t s, bool with_sum,
                          bool lat_frag) {
  const int G = share_slices(N, M);
  if (G == M / 32)
    hipLaunchKernelGGL((latent_share_kernel<R, 32>), dim3(N, G), dim3(256), 0, s, part, ntiles,
                       N * (B - 1), blk, am1, xh, w1p, mix_L, w_gate, w_up, w_down, B, M, V, dpart,
                       flags, pass);
  else
    hipLaunchKernelGGL((latent_share_kernel<R, 64>), dim3(N, G), dim3(256), 0, s, part, ntiles,
                       N * (B - 1), blk, am1, xh, w1p, mix_L, w_gate, w_up, w_down, B, M, V, dpart,
                       flags, pass);
  if (!with_sum) return hipGetLastError();
  constexpr int RPW = 256 / (R / 4);
  const dim3 grid(N, (B - 1 + RPW - 1) / RPW);
  if (G > 8)
    hipLaunchKernelGGL((latent_sum_kernel<R, 16>), grid, dim3(256), 0, s, dpart, B, G, lat, flags,
                       pass, part != nullptr ? 1 : 0, lat_frag ? 1 : 0);
  else
    hipLaunchKernelGGL((latent_sum_kernel<R, 8>), grid, dim3(256), 0, s, dpart, B, G, lat, flags,
                       pass, part != nullptr ? 1 : 0, lat_frag ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

// Slices of the share kernel per block: 32-unit slices while their N * M/32 workgroups fit one
// round on the 256 CUs (N <= 16 at M = 512), else 64-unit ones.
int share_slices(int N, int M) { return (int64_t)N * (M / 32) <= 256 ? M / 32 : M / 64; }

size_t latent_fused_scratch_bytes(int N, int r, int M) {
  return (size_t)N * share_slices(N, M) * 16 * r * sizeof(float);
}

hipError_t launch_latent_fused(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                               const float* xh, const float* w1p, const uint16_t* mix_L,
                               const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, int N, int B, int r, int M, int64_t V,
                               uint16_t* lat, float* dpart, int32_t* flags, int pass,
                               hipStream_t s, bool with_sum, bool lat_frag) {
  switch (r) {
    case 64: return launch_fused_r<64>(part, ntiles, blk, am1, xh, w1p, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, dpart, flags, pass, s, with_sum, lat_frag);
    case 128: return launch_fused_r<128>(part, ntiles, blk, am1, xh, w1p, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, dpart, flags, pass, s, with_sum, lat_frag);
    case 256: return launch_fused_r<256>(part, ntiles, blk, am1, xh, w1p, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, dpart, flags, pass, s, with_sum, lat_frag);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fold_embedding(const uint16_t* w1, const uint16_t* in_proj, int r, int64_t V,
                                 float* w1p, hipStream_t s) {
  const dim3 grid((unsigned)((V + 255) / 256));
  switch (r) {
    case 64: hipLaunchKernelGGL(fold_embedding_kernel<64>, grid, dim3(256), 0, s, w1, in_proj, V, w1p); break;
    case 128: hipLaunchKernelGGL(fold_embedding_kernel<128>, grid, dim3(256), 0, s, w1, in_proj, V, w1p); break;
    case 256: hipLaunchKernelGGL(fold_embedding_kernel<256>, grid, dim3(256), 0, s, w1, in_proj, V, w1p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t latent_scratch_bytes(int N, int r, int M) {
  const size_t nrows = (size_t)N * 16;
  return nrows * r * 4 + nrows * r * 2 + nrows * M * 2;
}

hipError_t launch_latent(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                         const float* xh, const uint16_t* w1, const uint16_t* in_proj,
                         const uint16_t* mix_L, const uint16_t* w_gate, const uint16_t* w_up,
                         const uint16_t* w_down, int N, int B, int r, int M, int64_t V,
                         uint16_t* lat, void* scratch, int32_t* flags, int pass, hipStream_t s,
                         bool lat_frag) {
  switch (r) {
    case 64: return launch_r<64>(part, ntiles, blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s, lat_frag);
    case 128: return launch_r<128>(part, ntiles, blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s, lat_frag);
    case 256: return launch_r<256>(part, ntiles, blk, am1, xh, w1, in_proj, mix_L, w_gate, w_up, w_down, N, B, M, V, lat, scratch, flags, pass, s, lat_frag);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xpress
