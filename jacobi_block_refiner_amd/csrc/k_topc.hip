// Top-C path of an XPress step (gfx950).
//
// Once per step (vLLM API page "vllm.model_executor.models.qwen3_xpress", top-C branch of
// jacobi_refine_greedy): each draft row's candidate set is the c = min(C, V) ids with the largest
// base logits, under the total order (value descending, id ascending), kept in ascending id
// order; base_c is gathered once and reused by every pass (and, for callers that want it, the
// readout rows w2c = w2[cand]).
// Per pass (vLLM API page "vllm.v1.worker.gpu.spec_decode.xpress.kernels",
// _xpress_topc_argmax_to_blk_kernel): the GEMV base_c + w2[cand] . lat, its argmax (lowest
// vocabulary id on ties) and the candidate -> vocabulary id -> blk write, in one kernel. A step
// reads the candidates' rows from w2 through their ids: no gathered copy (rows*c*r*2 bytes, 126
// MB at 480 rows of 512 candidates) and no gather launch, and 10% faster top-512 steps than
// reading the copy. The kernel also reads a caller's gathered w2c.
//
// Selection is a per-row radix select on the 16-bit order-preserving key of the bf16 value
// (high byte histogram, then low byte histogram inside the boundary bin), followed by one ordered
// compaction pass that keeps every id above the threshold key and the lowest-id ties at it.
#include "launch.hpp"
#include "hidden_tile.hpp"
#include "xpress_common.hpp"

#include <limits.h>

namespace xpress {

namespace {

// Larger key <=> larger value; -0.0 and +0.0 share a key.
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  b &= 0xffffu;
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS round trips): shifts
// by 1, 2, 4 and 8 lanes inside each 16-lane row, then lane 15 of rows 0 and 2 added into rows
// 1 and 3, and lane 31 into rows 2 and 3 (the GFX9 row broadcasts). Lanes whose source lies
// outside their row add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ int block_exclusive_scan(int x, int* s_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = s_tmp[w];
    if (w < wave) pre += t;
    total += t;
  }
  __syncthreads();
  return pre + inc - x;
}

__device__ __forceinline__ void load8_keys(const uint16_t* row, int64_t id0, int64_t V,
                                           uint32_t key[8], uint16_t bits[8]) {
  if (id0 + 8 <= V) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + id0);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bits[2 * e] = (uint16_t)(w[e] & 0xffffu);
      bits[2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) key[e] = order_key(bits[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = id0 + e < V;
      bits[e] = in ? row[id0 + e] : 0;
      key[e] = in ? order_key(bits[e]) : 0xffffffffu;  // never counted, never selected
    }
  }
}

// Exact selection of one row by a two-level radix select over the whole row, then an ordered
// compaction. Called by the whole workgroup (256 threads).
__device__ void select_row_exact(const uint16_t* __restrict__ row, int64_t V, int c,
                                 int64_t* __restrict__ out_id, uint16_t* __restrict__ out_b,
                                 uint32_t* s_hist, int* s_tmp, uint32_t* s_par) {
  const int tid = threadIdx.x;
  const int64_t nchunk = (V + 7) / 8;

  // pass 1: high byte histogram
  s_hist[tid] = 0;
  __syncthreads();
  for (int64_t q = tid; q < nchunk; q += 256) {
    uint32_t key[8];
    uint16_t bits[8];
    load8_keys(row, q * 8, V, key, bits);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (key[e] <= 0xffffu) atomicAdd(&s_hist[key[e] >> 8], 1u);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    int hb = 0;
    for (int b = 255; b >= 0; --b) {
      if (acc + s_hist[b] >= (uint32_t)c) { hb = b; break; }
      acc += s_hist[b];
    }
    s_par[0] = (uint32_t)hb;
    s_par[1] = acc;  // ids with a larger high byte
  }
  __syncthreads();
  const uint32_t h1 = s_par[0], above1 = s_par[1];
  s_hist[tid] = 0;
  __syncthreads();
  // pass 2: low byte histogram inside the boundary bin
  for (int64_t q = tid; q < nchunk; q += 256) {
    uint32_t key[8];
    uint16_t bits[8];
    load8_keys(row, q * 8, V, key, bits);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (key[e] <= 0xffffu && (key[e] >> 8) == h1) atomicAdd(&s_hist[key[e] & 0xffu], 1u);
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t rem = (uint32_t)c - above1;
    uint32_t acc = 0;
    int lb = 0;
    for (int b = 255; b >= 0; --b) {
      if (acc + s_hist[b] >= rem) { lb = b; break; }
      acc += s_hist[b];
    }
    s_par[2] = (h1 << 8) | (uint32_t)lb;   // threshold key T
    s_par[3] = (uint32_t)c - (above1 + acc);  // ids equal to T that are taken (lowest ids)
  }
  __syncthreads();
  const uint32_t T = s_par[2];
  const int need_eq = (int)s_par[3];

  // pass 3: ordered compaction, 2048 ids per round, ascending id order
  int eq_carry = 0, sel_carry = 0;
  for (int64_t id_base = 0; id_base < V && sel_carry < c; id_base += 2048) {
    const int64_t id0 = id_base + (int64_t)tid * 8;
    uint32_t key[8];
    uint16_t bits[8];
    if (id0 < V) {
      load8_keys(row, id0, V, key, bits);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { key[e] = 0xffffffffu; bits[e] = 0; }
    }
    int n_eq = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) n_eq += (key[e] == T);
    int eq_total;
    const int eq_before = eq_carry + block_exclusive_scan(n_eq, s_tmp, eq_total);
    bool sel[8];
    int n_sel = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool gt = key[e] <= 0xffffu && key[e] > T;
      const bool eq = key[e] == T;
      sel[e] = gt || (eq && eq_before + eq_seen < need_eq);
      eq_seen += eq;
      n_sel += sel[e];
    }
    int sel_total;
    const int pos0 = sel_carry + block_exclusive_scan(n_sel, s_tmp, sel_total);
    int k = pos0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (sel[e]) {
        if (k < c) {  // exactly c are taken; the bound only guards the row's storage
          out_id[k] = id0 + e;
          out_b[k] = bits[e];
        }
        ++k;
      }
    eq_carry += eq_total;
    sel_carry += sel_total;
  }
}

// Fast path for c <= 1024, exact. Each thread splits the ids it visits (in increasing order) into
// at most 8 groups and records each group's largest key: at most 2048 group maxima, which are
// distinct elements of the row. t0 = the c-th largest of them is then at most the c-th largest
// key of the row, so every element of the answer -- ties at the boundary included -- has a key
// >= t0. A second pass appends the elements with key >= t0 to an LDS buffer (at least c of them;
// if more than the buffer holds, the row falls back to select_row_exact), and the exact selection
// runs on the buffer: threshold by radix select, the boundary ties by id rank, and each winner
// written at its rank by id (ascending id order).
constexpr int kBuf = 2048;

// hist[bin] += 1 for every lane with `valid`, one LDS atomic per distinct bin in the wave: the
// lanes of the wave's smallest pending lane's bin are counted together (ballot) and leave the
// loop. Keys near the top of a row share a handful of high bytes, and plain per-lane atomics on
// the same bin serialize; the loop runs once per distinct bin (wave-uniform).
__device__ __forceinline__ void hist_add_aggregated(uint32_t* hist, int bin, bool valid) {
  const int lane = threadIdx.x & 63;
  uint64_t pending = __ballot(valid);
  while (pending) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int lb = __shfl(bin, leader);
    const uint64_t same = __ballot(bin == lb) & pending;
    if (lane == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    pending &= ~same;
  }
}
__device__ __forceinline__ uint32_t radix_kth(const uint32_t* keys, int n, int k, uint32_t* s_hist,
                                              uint32_t* s_par, int* s_tmp, uint32_t* above_out) {
  // keys: 17-bit (key + 1, 0 = empty); returns the k-th largest non-empty key (as key + 1) and
  // sets *above_out = number of keys strictly above it; with fewer than k non-empty keys it
  // returns 0. Whole workgroup (256 threads). Two histogram levels over the 16-bit key (high
  // byte, then low byte inside the boundary bin); the boundary bin is found by a parallel scan
  // over the bins in descending order: thread t owns bin 255 - t, and the bin whose [count above,
  // count above + own count) holds k - 1 is the one.
  const int tid = threadIdx.x;
  s_hist[tid] = 0;
  __syncthreads();
  for (int j0 = 0; j0 < n; j0 += 256) {  // uniform trip count (n is a multiple of 256)
    const uint32_t k1 = keys[j0 + tid];
    hist_add_aggregated(s_hist, (int)((k1 - 1) >> 8) & 255, k1 != 0);
  }
  __syncthreads();
  int total;
  {
    const int bin = 255 - tid;
    const int cnt = (int)s_hist[bin];
    const int above = block_exclusive_scan(cnt, s_tmp, total);
    if (above < k && k <= above + cnt) {
      s_par[0] = (uint32_t)bin;
      s_par[1] = (uint32_t)above;
    }
  }
  if (total < k) {  // uniform: fewer than k non-empty keys
    *above_out = (uint32_t)total;
    return 0u;
  }
  __syncthreads();
  const uint32_t h1 = s_par[0], a1 = s_par[1];
  s_hist[tid] = 0;
  __syncthreads();
  for (int j = tid; j < n; j += 256) {
    const uint32_t k1 = keys[j];
    if (k1 && ((k1 - 1) >> 8) == h1) atomicAdd(&s_hist[(k1 - 1) & 0xffu], 1u);
  }
  __syncthreads();
  {
    const int rem = k - (int)a1;
    const int bin = 255 - tid;
    const int cnt = (int)s_hist[bin];
    const int above = block_exclusive_scan(cnt, s_tmp, total);
    if (above < rem && rem <= above + cnt) {
      s_par[2] = ((h1 << 8) | (uint32_t)bin) + 1;
      s_par[3] = a1 + (uint32_t)above;
    }
  }
  __syncthreads();
  const uint32_t t = s_par[2];
  *above_out = s_par[3];
  __syncthreads();
  return t;
}

// LDS of one row's selection (the caller's, so that a launch with other work can overlay it).
// The chunk maxima of a row of up to kCmaxLds chunks (153,600 ids) stay in LDS from the first pass
// to the chunk list, where the buffer's ids and values later go; longer rows keep them in the
// caller's global buffer. The chunk list holds at most kBuf chunks: each listed chunk holds an
// element of the buffer, so a longer list would overflow the buffer anyway.
constexpr int kCmaxLds = 19200;
struct alignas(16) SelLds {
  uint32_t hist[256];
  int tmp[4];
  uint32_t par[4];
  int tmp_r[4];        // radix_kth's scan
  uint32_t key[kBuf];  // key + 1 (0: empty)
  union alignas(16) Shared {
    struct {
      int id[kBuf];
      uint16_t bits[kBuf];  // the buffered values' bf16 bits
    } buf;
    uint16_t cmax[kCmaxLds];  // bf16 bits of the chunk maxima (first pass to chunk list)
  } u;
  uint16_t hc[kBuf];    // chunks whose maximum can hold an answer, ascending
  uint32_t bk[4];       // the starting block's per-wave winners (key + 1, id)
  int bi[4];
  float bv[4];
};

// Returns whether the buffered path ran; then, with start_slot given, the row's best id (largest
// value, lowest id) has been written there from the buffer.
__device__ __forceinline__ bool topc_select_row(int p, const uint16_t* __restrict__ base,
                                                int64_t ld, int64_t V, int c,
                                                int64_t* __restrict__ cand,
                                                uint16_t* __restrict__ base_c,
                                                uint16_t* __restrict__ cmax, SelLds& L,
                                                int64_t* __restrict__ start_slot) {
  uint32_t* s_hist = L.hist;
  int* s_tmp = L.tmp;
  uint32_t* s_par = L.par;
  uint32_t* s_key = L.key;
  int* s_id = L.u.buf.id;
  uint16_t* s_bits = L.u.buf.bits;
  uint16_t* s_hc = L.hc;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint16_t* row = base + (int64_t)p * ld;
  int64_t* out_id = cand + (int64_t)p * c;
  uint16_t* out_b = base_c + (int64_t)p * c;
  const int64_t nchunk = (V + 7) / 8;
  const int64_t nchunk8 = (nchunk + 7) / 8 * 8;
  const bool cm_lds = nchunk8 <= kCmaxLds;  // the chunk maxima in LDS (else in `cmax`)
  // the chunk list holds 16-bit chunk indexes; without chunk maxima (a long row and no
  // workspace) the exact whole-row path runs
  if (c > 1024 || nchunk > 65536 || (!cm_lds && cmax == nullptr)) {
    select_row_exact(row, V, c, out_id, out_b, s_hist, s_tmp, s_par);
    return false;
  }
  // The two passes over the row load kLB chunks per thread before using any of them, so enough
  // bytes are in flight to stream the row (one chunk at a time is latency-bound). Rows are padded
  // to the stride, so the last chunk is read whole. The passes compare values as fp32 (a bf16
  // widens exactly; the order of the finite values is the key order, -0.0 equal to +0.0), and ids
  // >= V, or chunks past the row, read as -inf, below every finite value.
  constexpr int kLB = 8;
  const uint4* row4 = reinterpret_cast<const uint4*>(row);
  auto load_batch = [&](int64_t q0, uint4 (&raw)[kLB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      const int64_t q = q0 + 256 * u;
      raw[u] = q < nchunk ? row4[q] : make_uint4(0, 0, 0, 0);
    }
  };
  auto widen = [&](int64_t q, const uint4& raw, float (&x)[8]) __attribute__((always_inline)) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
    if (q * 8 + 8 > V) {  // the row's last chunk, or past it
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (q * 8 + e >= V) x[e] = -INFINITY;
    }
  };
  // key + 1 of a finite fp32 that holds a bf16 value
  auto key1_of = [](float v) __attribute__((always_inline)) {
    return order_key(__float_as_uint(v) >> 16) + 1;
  };
  // chunk maxima (bf16 bits), written by pass 1 and read back by pass 3 so that it re-reads only
  // the chunks that can hold an answer
  uint16_t* cmax_row = cm_lds ? nullptr : cmax + (int64_t)p * nchunk8;
  uint16_t* s_cm = L.u.cmax;
  // 1. group maxima: thread tid visits chunks tid + 256 i; groups of gv visits (<= 8 groups)
  const int nv_max = (int)((nchunk + 255) / 256);
  const int gv = (nv_max + 7) / 8;
  {
    float gm = -INFINITY;
    int g = 0, inside = 0;
    for (int64_t q0 = tid; q0 < nchunk; q0 += 256 * kLB) {
      uint4 raw[kLB];
      load_batch(q0, raw);
#pragma unroll
      for (int u = 0; u < kLB; ++u) {
        const int64_t q = q0 + 256 * u;
        if (q < nchunk) {
          float x[8];
          widen(q, raw[u], x);
          const float cm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
          const uint16_t cb = (uint16_t)(__float_as_uint(cm) >> 16);  // -inf: 0xff80
          if (cm_lds)
            s_cm[q] = cb;
          else
            cmax_row[q] = cb;
          gm = fmaxf(gm, cm);
          if (++inside == gv) {
            s_key[tid * 8 + g] = gm > -INFINITY ? key1_of(gm) : 0u;
            ++g;
            inside = 0;
            gm = -INFINITY;
          }
        }
      }
    }
    if (inside) s_key[tid * 8 + g++] = gm > -INFINITY ? key1_of(gm) : 0u;
    for (; g < 8; ++g) s_key[tid * 8 + g] = 0;
    for (int64_t q = nchunk + tid; q < nchunk8; q += 256) {  // padding to 8 chunk maxima: -inf
      if (cm_lds)
        s_cm[q] = 0xff80u;
      else
        cmax_row[q] = 0xff80u;
    }
  }
  __threadfence_block();
  __syncthreads();
  // 2. t0: the c-th largest group maximum (every group maximum is non-empty if its group had an
  // id below V; with fewer than c of them t0 = 0, below every key)
  uint32_t above;
  const uint32_t t0 = radix_kth(s_key, kBuf, c, s_hist, s_par, L.tmp_r, &above);
  // the smallest fp32 value with key >= t0 - 1 (any finite value when t0 <= 1: the key's bf16
  // bits, inverse of order_key, would not be a finite value then)
  float v0 = -3.4028235e38f;
  if (t0 > 1) {
    const uint32_t k = t0 - 1;
    const uint32_t bits = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
    v0 = fmaxf(__uint_as_float(bits << 16), -3.4028235e38f);
  }
  for (int j = tid; j < kBuf; j += 256) s_key[j] = 0;
  __syncthreads();
  // 3. Every element with value >= v0 into the buffer, in ascending id order.
  // 3a. The chunks whose maximum reaches v0, listed in ascending order: per round, thread tid takes
  // the kLB consecutive groups of 8 chunk maxima g0 + kLB*tid .. +kLB-1 (128 contiguous bytes,
  // all read before any is used); one block-wide exclusive scan of the threads' hit counts places
  // each thread's hits, in ascending order, after those of the lower threads (two rounds per row
  // of 151936 ids). A list that would overflow sends the row to the exact path.
  const int64_t n8 = nchunk8 / 8;
  const uint4* cm4 = reinterpret_cast<const uint4*>(cmax_row);
  const uint4* s_cm4 = reinterpret_cast<const uint4*>(s_cm);
  int nhc = 0;  // uniform
  for (int64_t g0 = 0; g0 < n8; g0 += 256 * kLB) {
    uint4 m8[kLB];
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      const int64_t g = g0 + kLB * tid + u;
      const bool in = g < n8;
      const int64_t gc = in ? g : 0;
      m8[u] = cm_lds ? s_cm4[gc] : cm4[gc];
      if (!in) m8[u] = make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
    }
    uint64_t hm = 0;  // bit 8u + e: chunk 8 (g0 + kLB*tid + u) + e reaches v0
#pragma unroll
    for (int u = 0; u < kLB; ++u) {
      const uint32_t w[4] = {m8[u].x, m8[u].y, m8[u].z, m8[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bv = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
        hm |= (uint64_t)(__uint_as_float(bv) >= v0 ? 1u : 0u) << (8 * u + e);
      }
    }
    int tot;
    int pos = nhc + block_exclusive_scan(__popcll(hm), s_tmp, tot);
    const int64_t c0 = (g0 + kLB * tid) * 8;
    while (hm) {  // the thread's hits in ascending order
      const int bit = __ffsll((unsigned long long)hm) - 1;
      if (pos < kBuf) s_hc[pos] = (uint16_t)(c0 + bit);
      ++pos;
      hm &= hm - 1;
    }
    nhc += tot;
  }
  if (nhc > kBuf) {  // uniform
    select_row_exact(row, V, c, out_id, out_b, s_hist, s_tmp, s_par);
    return false;
  }
  __syncthreads();  // the list is complete (and the chunk maxima, which share LDS with the
                    // buffer's ids and values, are no longer read)
  // 3b. The listed chunks' elements >= v0 appended in list order (ascending ids): per round,
  // thread tid reads chunk tid of the round (up to four rounds' reads issued together), and a
  // block-wide scan places its hits. More than kBuf of them, or fewer than c, sends the row to the
  // exact path.
  int nbuf = 0;  // uniform
  for (int i0 = 0; i0 < nhc; i0 += 4 * 256) {
    uint4 raw[4];
    int64_t qs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 256 * u + tid;
      qs[u] = i < nhc ? s_hc[i] : nchunk;  // past the list: a chunk past the row, all -inf
      raw[u] = i < nhc ? row4[qs[u]] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + 256 * u >= nhc) break;  // uniform
      float x[8];
      widen(qs[u], raw[u], x);
      uint32_t hm = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) hm |= (x[e] >= v0 ? 1u : 0u) << e;
      int tot;
      int pos = nbuf + block_exclusive_scan(__popc(hm), s_tmp, tot);
      const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((hm >> e) & 1u) {
          if (pos < kBuf) {
            s_key[pos] = key1_of(x[e]);
            s_id[pos] = (int)(qs[u] * 8 + e);
            s_bits[pos] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
          }
          ++pos;
        }
      nbuf += tot;
    }
  }
  // -inf and NaN never pass the compare, so a row with fewer than c finite values has fewer than
  // c buffered elements; the exact path orders every bit pattern by its key
  if (nbuf > kBuf || nbuf < c) {  // uniform
    select_row_exact(row, V, c, out_id, out_b, s_hist, s_tmp, s_par);
    return false;
  }
  __syncthreads();
  // 4. The threshold T (c-th largest key of the buffer; empty slots are 0), then one ordered
  // compaction: thread tid owns buffer slots 8*tid .. 8*tid+7; every key above T is taken, and of
  // the keys equal to T the first need_eq in buffer order, the lowest ids. Written in buffer order:
  // ascending ids.
  const uint32_t T = radix_kth(s_key, kBuf, c, s_hist, s_par, L.tmp_r, &above);
  const int need_eq = c - (int)above;
  uint32_t k8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) k8[e] = s_key[8 * tid + e];
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) n_eq += k8[e] == T;
  int eq_tot;
  int eq_rank = block_exclusive_scan(n_eq, s_tmp, eq_tot);
  uint32_t sm = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bool take = k8[e] > T;
    if (k8[e] == T) take = eq_rank++ < need_eq;
    sm |= (take ? 1u : 0u) << e;
  }
  int sel_tot;
  int pos = block_exclusive_scan(__popc(sm), s_tmp, sel_tot);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((sm >> e) & 1u) {
      if (pos < c) {  // exactly c are taken; the bound only guards the row's storage
        out_id[pos] = s_id[8 * tid + e];
        out_b[pos] = s_bits[8 * tid + e];
      }
      ++pos;
    }
  if (start_slot) {  // uniform: the best buffered element (largest key, lowest id)
    const int wave = tid >> 6;
    uint32_t bk = 0;
    int bid = INT_MAX;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int id = s_id[8 * tid + e];
      const bool take = k8[e] > bk || (k8[e] != 0 && k8[e] == bk && id < bid);
      bk = take ? k8[e] : bk;
      bid = take ? id : bid;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t ok = (uint32_t)__shfl_xor((int)bk, off);
      const int oi = __shfl_xor(bid, off);
      const bool take = ok > bk || (ok != 0 && ok == bk && oi < bid);
      bk = take ? ok : bk;
      bid = take ? oi : bid;
    }
    if (lane == 0) {
      L.bk[wave] = bk;
      L.bi[wave] = bid;
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const bool take = L.bk[w] > bk || (L.bk[w] != 0 && L.bk[w] == bk && L.bi[w] < bid);
        bk = take ? L.bk[w] : bk;
        bid = take ? L.bi[w] : bid;
      }
      *start_slot = bid;
    }
  }
  return true;
}

// Draft row p, by one workgroup: the row's candidate set; with blk given, also the row's starting
// token (vLLM API page "vllm.model_executor.models.qwen3_xpress", jacobi_refine_greedy: the
// argmax of the base logits, lowest id on ties), which is the best of the candidates under the
// same order, written into blk[n, 1 + p % (B - 1)] (and the anchor into slot 0): the starting
// block without a separate pass over base.
__device__ __forceinline__ void topc_select_block(int p, const uint16_t* __restrict__ base,
                                                  int64_t ld, int64_t V, int c,
                                                  int64_t* __restrict__ cand,
                                                  uint16_t* __restrict__ base_c,
                                                  const int64_t* __restrict__ anchor,
                                                  int64_t* __restrict__ blk, int B,
                                                  uint16_t* __restrict__ cmax, SelLds& L) {
  int64_t* slot = blk ? blk + (int64_t)(p / (B - 1)) * B + 1 + p % (B - 1) : nullptr;
  const bool buffered = topc_select_row(p, base, ld, V, c, cand, base_c, cmax, L, slot);
  if (!blk) return;
  // the block's first row also stores the anchor in slot 0
  if (p % (B - 1) == 0 && threadIdx.x == 0) blk[(int64_t)(p / (B - 1)) * B] = anchor[p / (B - 1)];
  if (buffered) return;  // uniform: the starting token is written
  // the exact path: the best of the candidates it wrote
  float* s_bv = L.bv;
  int* s_bi = L.bi;
  __threadfence_block();
  __syncthreads();  // the row's candidates and values are written (by this workgroup)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t* ids = cand + (int64_t)p * c;
  const uint16_t* vals = base_c + (int64_t)p * c;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int k = tid; k < c; k += 256) argmax_merge(bv, bi, __uint_as_float((uint32_t)vals[k] << 16), (int)ids[k]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    argmax_merge(bv, bi, ov, oi);
  }
  if (lane == 0) {
    s_bv[wave] = bv;
    s_bi[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, s_bv[w], s_bi[w]);
    *slot = bi;
  }
}

__global__ __launch_bounds__(256) void topc_select_kernel(const uint16_t* __restrict__ base,
                                                          int64_t ld, int64_t V, int c,
                                                          int64_t* __restrict__ cand,
                                                          uint16_t* __restrict__ base_c,
                                                          const int64_t* __restrict__ anchor,
                                                          int64_t* __restrict__ blk, int B,
                                                          uint16_t* __restrict__ cmax) {
  __shared__ SelLds lds;
  topc_select_block(blockIdx.x, base, ld, V, c, cand, base_c, anchor, blk, B, cmax, lds);
}

// The start of a top-C step in one launch: workgroups [0, g1) are the hidden GEMM's tiles (mt x
// nt tiles per split, split-major), the rest the draft rows' selection. The two are independent;
// the GEMM is latency-bound and hides behind the selection. The two roles overlay one LDS area
// and the GEMM keeps 4 k chunks in flight, so a CU holds three of these workgroups and the whole
// launch (256 tiles + 480 rows at 32 blocks) runs in one round.
__global__ __launch_bounds__(256) void topc_start_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ down_h,
    const uint16_t* __restrict__ down_g, int NB, int H, int r, int kslice,
    float* __restrict__ part, int g1, int mt, int nt, const uint16_t* __restrict__ base,
    int64_t ld, int64_t V, int c, int64_t* __restrict__ cand, uint16_t* __restrict__ base_c,
    const int64_t* __restrict__ anchor, int64_t* __restrict__ blk, int B,
    uint16_t* __restrict__ cmax, int32_t* __restrict__ zero_flags, int nzero) {
  const int i = blockIdx.x;
  if (zero_flags && i == 0)  // the step's pass flags (read only by later launches)
    for (int q = threadIdx.x; q < nzero; q += blockDim.x) zero_flags[q] = 0;
  __shared__ union {
    GemmLds gemm;
    SelLds sel;
  } lds;
  if (i < g1)
    hidden_gemm_tile<4>(h, down_h, down_g, NB, H, r, kslice, part, i % mt, (i / mt) % nt, i / (mt * nt), lds.gemm);
  else
    topc_select_block(i - g1, base, ld, V, c, cand, base_c, anchor, blk, B, cmax, lds.sel);
}

__global__ __launch_bounds__(256) void topc_gather_kernel(const int64_t* __restrict__ cand,
                                                          const uint16_t* __restrict__ w2,
                                                          int64_t total, int rq,
                                                          uint16_t* __restrict__ w2c) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t pk = i / rq;
  const int q = (int)(i % rq);
  const int64_t id = cand[pk];
  reinterpret_cast<uint4*>(w2c)[i] = reinterpret_cast<const uint4*>(w2)[id * rq + q];
}

// One workgroup per draft row. Lanes form groups of G = R/8 that each hold one candidate's row
// (16 bytes per lane, so a load reads whole 512-byte rows); the group's partial dot products are
// summed with xor shuffles. Each lane keeps U loads in flight per round (the rows stream once
// per pass: the kernel is bound by how many bytes are in flight). BY_ID: the rows are w2[cand[p,
// k]] (table = w2 [V, r]), and each lane loads the ids of its next round's candidates one round
// ahead; otherwise table = w2c [rows, c, r], the gathered copy. The winner is tracked by
// (value, vocabulary id): equal values go to the lowest id whatever the order of cand.
template <int R, bool BY_ID>
__global__ __launch_bounds__(256) void topc_readout_kernel(
    const uint16_t* __restrict__ lat, const float* __restrict__ shares, int nsh,
    const uint16_t* __restrict__ table, const uint16_t* __restrict__ base_c,
    const int64_t* __restrict__ cand, int B, int c, int64_t* __restrict__ blk, int32_t* changed,
    int32_t* flags, int pass) {
  if (pass_skipped(flags, pass)) return;
  constexpr int G = R / 8;        // lanes per candidate
  constexpr int CPW = 64 / G;     // candidates per wave per load
  // loads in flight per lane: gathered rows 4 (2, 3, 6, 8 and 16 measured slower); rows through
  // the ids 6 (4: 10% slower whole top-512 steps, 5 the same, 7 and 8 slower)
  constexpr int U = BY_ID ? 6 : 4;
  constexpr int CPR = 4 * CPW * U;  // candidates per workgroup round
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane % G, sub = lane / G;
  const uint16_t* bc = base_c + (int64_t)p * c;
  float lv[8];
  if (shares) {
    // The latent row from the nsh slice shares of the latent kernels ([N, nsh, 16, r] fp32, the
    // residual in share 0), summed in slice order and rounded to bf16 exactly as the sum kernel
    // forms lat (the values are the same bits).
    const int n = p / (B - 1), b = 1 + p % (B - 1);
    const float4* sp = reinterpret_cast<const float4*>(shares + ((int64_t)n * nsh * 16 + b) * R) + 2 * q;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < nsh; g0 += 8) {
      float4 v[8][2];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t off = (int64_t)min(g0 + k, nsh - 1) * 16 * (R / 4);
        v[k][0] = sp[off];
        v[k][1] = sp[off + 1];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool on = g0 + k < nsh;
        a[0] += on ? v[k][0].x : 0.f; a[1] += on ? v[k][0].y : 0.f;
        a[2] += on ? v[k][0].z : 0.f; a[3] += on ? v[k][0].w : 0.f;
        a[4] += on ? v[k][1].x : 0.f; a[5] += on ? v[k][1].y : 0.f;
        a[6] += on ? v[k][1].z : 0.f; a[7] += on ? v[k][1].w : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) lv[e] = bf16_to_f32(f32_to_bf16(a[e]));
  } else {
    const uint4 u = reinterpret_cast<const uint4*>(lat + (int64_t)p * R)[q];
    lv[0] = bf16_lo(u.x); lv[1] = bf16_hi(u.x); lv[2] = bf16_lo(u.y); lv[3] = bf16_hi(u.y);
    lv[4] = bf16_lo(u.z); lv[5] = bf16_hi(u.z); lv[6] = bf16_lo(u.w); lv[7] = bf16_hi(u.w);
  }
  // BY_ID: the whole table, indexed by vocabulary id; otherwise this row's gathered rows
  const uint4* wrow = reinterpret_cast<const uint4*>(table + (BY_ID ? 0 : (int64_t)p * c * R));
  const int64_t* crow = cand + (int64_t)p * c;
  float bv = -INFINITY;
  int bid = INT_MAX;  // vocabulary id of the best candidate so far
  int idn[U];         // BY_ID: the ids of this lane's candidates in the coming round
  if constexpr (BY_ID) {
#pragma unroll
    for (int j = 0; j < U; ++j) idn[j] = (int)crow[min((j * 4 + wave) * CPW + sub, c - 1)];
  }
  for (int k0 = 0; k0 < c; k0 += CPR) {
    uint4 u[U];
    uint16_t bk16[U];
    int idc[U];  // this round's ids
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int k = min(k0 + (j * 4 + wave) * CPW + sub, c - 1);  // past c: repeats, masked
      idc[j] = BY_ID ? idn[j] : (int)crow[k];
      u[j] = wrow[(BY_ID ? (int64_t)idn[j] : (int64_t)k) * G + q];
      bk16[j] = bc[k];
    }
    if constexpr (BY_ID) {  // the next round's ids (past c: clamped, unused)
#pragma unroll
      for (int j = 0; j < U; ++j) idn[j] = (int)crow[min(k0 + CPR + (j * 4 + wave) * CPW + sub, c - 1)];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      float d = lv[0] * bf16_lo(u[j].x);
      d = fmaf(lv[1], bf16_hi(u[j].x), d);
      d = fmaf(lv[2], bf16_lo(u[j].y), d);
      d = fmaf(lv[3], bf16_hi(u[j].y), d);
      d = fmaf(lv[4], bf16_lo(u[j].z), d);
      d = fmaf(lv[5], bf16_hi(u[j].z), d);
      d = fmaf(lv[6], bf16_lo(u[j].w), d);
      d = fmaf(lv[7], bf16_hi(u[j].w), d);
#pragma unroll
      for (int off = G / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      const int k = k0 + (j * 4 + wave) * CPW + sub;
      const bool in = k < c;
      argmax_merge(bv, bid, in ? bf16_to_f32(bk16[j]) + d : -INFINITY, in ? idc[j] : INT_MAX);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bid, off);
    argmax_merge(bv, bid, ov, oi);
  }
  if (lane == 0) {
    s_v[wave] = bv;
    s_i[wave] = bid;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bid, s_v[w], s_i[w]);
    // a row whose every logit is NaN merges nothing: take its first candidate (results for
    // non-finite inputs are unspecified, but the id stays a candidate's)
    const int64_t id = bid == INT_MAX ? crow[0] : (int64_t)bid;
    const int n = p / (B - 1), b = 1 + p % (B - 1);
    int64_t* slot = blk + (int64_t)n * B + b;
    if (*slot != id) {
      *slot = id;
      if (changed) __hip_atomic_store(changed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (flags) __hip_atomic_store(flags + pass, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_topc_select(const uint16_t* base, int64_t ld, int rows, int64_t V, int c,
                              int64_t* cand, uint16_t* base_c, const int64_t* anchor,
                              int64_t* blk, int B, uint16_t* cmax, hipStream_t s) {
  hipLaunchKernelGGL(topc_select_kernel, dim3(rows), dim3(256), 0, s, base, ld, V, c, cand, base_c,
                     anchor, blk, B, cmax);
  return hipGetLastError();
}

hipError_t launch_topc_start(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                             int NB, int H, int r, float* part, const uint16_t* base, int64_t ld,
                             int rows, int64_t V, int c, int64_t* cand, uint16_t* base_c,
                             const int64_t* anchor, int64_t* blk, int B, uint16_t* cmax,
                             hipStream_t s, int32_t* zero_flags, int nzero) {
  const int ns = hidden_splits(NB, H, r);
  const int kslice = hidden_chunks_per_split(NB, H, r) * kTK;
  const int mt = (NB + kTM - 1) / kTM, nt = (2 * r) / kTN;
  const int g1 = mt * nt * ns;
  hipLaunchKernelGGL(topc_start_kernel, dim3((unsigned)(g1 + rows)), dim3(256), 0, s, h, down_h,
                     down_g, NB, H, r, kslice, part, g1, mt, nt, base, ld, V, c, cand, base_c,
                     anchor, blk, B, cmax, zero_flags, nzero);
  return hipGetLastError();
}

size_t topc_select_scratch_bytes(int rows, int64_t V) {
  const int64_t nchunk = (V + 7) / 8;
  const int64_t nchunk8 = (nchunk + 7) / 8 * 8;
  // short rows keep their chunk maxima in LDS; rows past 65536 chunks take the exact path
  if (nchunk8 <= kCmaxLds || nchunk > 65536) return 0;
  return (size_t)rows * (size_t)nchunk8 * 2;
}

hipError_t launch_topc_gather(const int64_t* cand, const uint16_t* w2, int rows, int c, int r,
                              uint16_t* w2c, hipStream_t s) {
  const int rq = r / 8;
  const int64_t total = (int64_t)rows * c * rq;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(topc_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, cand, w2, total,
                     rq, w2c);
  return hipGetLastError();
}

template <bool BY_ID>
hipError_t launch_readout_t(const uint16_t* lat, const float* shares, int nsh,
                            const uint16_t* table, const uint16_t* base_c, const int64_t* cand,
                            int rows, int B, int r, int c, int64_t* blk, int32_t* changed,
                            int32_t* flags, int pass, hipStream_t s) {
  switch (r) {
    case 64:
      hipLaunchKernelGGL((topc_readout_kernel<64, BY_ID>), dim3(rows), dim3(256), 0, s, lat,
                         shares, nsh, table, base_c, cand, B, c, blk, changed, flags, pass);
      break;
    case 128:
      hipLaunchKernelGGL((topc_readout_kernel<128, BY_ID>), dim3(rows), dim3(256), 0, s, lat,
                         shares, nsh, table, base_c, cand, B, c, blk, changed, flags, pass);
      break;
    case 256:
      hipLaunchKernelGGL((topc_readout_kernel<256, BY_ID>), dim3(rows), dim3(256), 0, s, lat,
                         shares, nsh, table, base_c, cand, B, c, blk, changed, flags, pass);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topc_readout(const uint16_t* lat, const float* shares, int nsh,
                               const uint16_t* table, bool by_id, const uint16_t* base_c,
                               const int64_t* cand, int rows, int B, int r, int c, int64_t* blk,
                               int32_t* changed, int32_t* flags, int pass, hipStream_t s) {
  return by_id ? launch_readout_t<true>(lat, shares, nsh, table, base_c, cand, rows, B, r, c, blk,
                                        changed, flags, pass, s)
               : launch_readout_t<false>(lat, shares, nsh, table, base_c, cand, rows, B, r, c,
                                         blk, changed, flags, pass, s);
}

}  // namespace xpress
