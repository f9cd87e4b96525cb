// C ABI of the XPress pass library: argument checks, workspace carving and kernel sequencing.
// Every entry point validates on the host, then only enqueues kernels on the caller's stream.
#include "xpress.h"

#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "launch.hpp"

namespace {

// Scratch is sized for the widest supported MLP (M = 1024) and hidden size, so
// xpress_workspace_size does not depend on M or H.
constexpr int kMaxM = 1024;
constexpr int kMaxH = 16384;

thread_local std::string g_err;

xpress_status fail(xpress_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

xpress_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(XPRESS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return XPRESS_OK;
}

#define XP_TRY(expr, what)                                   \
  do {                                                       \
    xpress_status st_ = hip_check((expr), (what));           \
    if (st_ != XPRESS_OK) return st_;                        \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The readout's base copies address 16 rows from one scalar pointer with 32-bit lane offsets.
constexpr int64_t kMaxBaseLd = (int64_t)1 << 27;

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

xpress_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(XPRESS_ERR_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(XPRESS_ERR_ARG, "%s is not 16-byte aligned", name);
  return XPRESS_OK;
}

#define XP_PTR(p)                                        \
  do {                                                   \
    xpress_status st_ = check_ptr((p), #p);              \
    if (st_ != XPRESS_OK) return st_;                    \
  } while (0)

xpress_status check_dims(int B, int r, int64_t V) {
  if (B < 2 || B > 16) return fail(XPRESS_ERR_ARG, "B=%d outside [2, 16]", B);
  if (r != 64 && r != 128 && r != 256) return fail(XPRESS_ERR_ARG, "r=%d not in {64,128,256}", r);
  if (V < 1 || V * (int64_t)r >= ((int64_t)1 << 31))
    return fail(XPRESS_ERR_ARG, "V=%lld outside [1, 2^31/r)", (long long)V);
  return XPRESS_OK;
}

xpress_status check_weights(const xpress_weights* w, bool need_hidden, bool need_latent,
                            bool need_w2) {
  if (w == nullptr) return fail(XPRESS_ERR_ARG, "weights struct is NULL");
  xpress_status st = check_dims(w->B, w->r, w->V);
  if (st != XPRESS_OK) return st;
  if (need_hidden) {
    if (w->H < 64 || w->H % 64 || w->H > kMaxH)
      return fail(XPRESS_ERR_ARG, "H=%d not a multiple of 64 in [64, %d]", w->H, kMaxH);
    XP_PTR(w->down_h);
    XP_PTR(w->down_g);
    XP_PTR(w->in_proj);
  }
  if (need_latent) {
    const int M = w->M;
    if (M != 64 && M != 128 && M != 256 && M != 512 && M != 1024)
      return fail(XPRESS_ERR_ARG, "M=%d not in {64,128,256,512,1024}", M);
    XP_PTR(w->w1);
    XP_PTR(w->in_proj);
    XP_PTR(w->mix_L);
    XP_PTR(w->w_gate);
    XP_PTR(w->w_up);
    XP_PTR(w->w_down);
    if (w->w1p != nullptr && !aligned16(w->w1p))
      return fail(XPRESS_ERR_ARG, "w->w1p is not 16-byte aligned");
  }
  if (need_w2) XP_PTR(w->w2);
  return XPRESS_OK;
}

xpress_status check_layout(uint32_t lat_layout) {
  if (lat_layout != XPRESS_LAT_ROWS && lat_layout != XPRESS_LAT_FRAGMENTS)
    return fail(XPRESS_ERR_ARG, "lat_layout=%u is neither XPRESS_LAT_ROWS nor XPRESS_LAT_FRAGMENTS",
                lat_layout);
  return XPRESS_OK;
}

xpress_status check_base(const xpress_bf16* base, int64_t ld, int64_t V) {
  XP_PTR(base);
  if (ld < V || ld % 8 || ld > kMaxBaseLd)
    return fail(XPRESS_ERR_ARG, "base_ld=%lld must be >= V=%lld, a multiple of 8 and at most 2^27",
                (long long)ld, (long long)V);
  return XPRESS_OK;
}

// Whether the latent stage runs from the projected embedding table (share + sum kernels): while
// its N * M/64 share workgroups (one per block and 64-unit slice) number at most 448. Two of them
// fit on a CU, so up to 512 run in one round. Whole steps at M = 512: the table path is faster up
// to 56 blocks (16.8k against 15.7k passes/s at 32, 15.5k against 15.1k at 33, 12.0k against
// 11.8k at 40, 9.86k against 9.78k at 56) and the three-kernel path from 64 (9.48k against 9.26k
// at 64, 6.38k against 6.27k at 96, 5.10k against 4.97k at 128); it is taken there even when the
// table is given. The results agree within fp32 rounding either way.
constexpr int kTableMaxWorkgroups = 448;
bool table_fits(int N, int M) { return (int64_t)N * (M / 64) <= kTableMaxWorkgroups; }
bool use_table(const xpress_weights* w, int N) { return w->w1p != nullptr && table_fits(N, w->M); }

// Scratch of the latent stage for any M: the three-kernel path's, or the projected-table path's
// (slice shares) where some M lets that path run.
size_t latent_bytes(int N, int r) {
  size_t t = xpress::latent_scratch_bytes(N, r, kMaxM);
  for (int M = 64; M <= kMaxM; M *= 2) {
    const size_t b = table_fits(N, M) ? xpress::latent_fused_scratch_bytes(N, r, M) : 0;
    t = b > t ? b : t;
  }
  return t;
}

// Workspace regions of a call with N blocks.
struct Layout {
  size_t hdg = 0, xh = 0, lat = 0, lscr = 0, part = 0, flags = 0, cand = 0, base_c = 0,
         cmax = 0, total = 0;
};

Layout step_layout(int N, int B, int r, int H, int64_t V, int C, int K) {
  Layout L;
  const size_t rows = (size_t)N * (B - 1);
  const size_t c = C > 0 ? (size_t)(C < V ? C : V) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  (void)H;
  L.hdg = take(xpress::hidden_scratch_bytes_any_h(N * B, r));
  L.xh = take((size_t)N * B * r * sizeof(float));
  L.lat = take((rows + 31) / 32 * 32 * (size_t)r * 2);  // whole 32-row tiles (fragment order)
  L.lscr = take(latent_bytes(N, r));
  // sized for the largest range count (the count at one row chunk)
  L.part = take(C > 0 ? 0 : rows * (size_t)xpress::readout_tiles(V, 1) * sizeof(uint2));
  L.flags = take((size_t)(K + 1) * sizeof(int32_t));
  L.cand = take(rows * c * sizeof(int64_t));
  L.base_c = take(rows * c * 2);
  L.cmax = take(C > 0 ? xpress::topc_select_scratch_bytes((int)rows, V) : 0);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Library-owned workspace of the allocation-free step: one array per GPU, in the code object's
// device globals, held until the process ends. 64 MiB covers a full-vocabulary or top-512 step of
// up to 256 blocks (43.4 and 54.6 MiB at B = 16, r = 256, V = 151936, K = 15). In host code the name `scratch` is only a stand-in for the symbol; its device
// address on each GPU comes from hipGetSymbolAddress (scratch_ptr) and is what the kernels get.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device (the first call
// on it) with that device current.
xpress_status scratch_ptr(void** out) {
  int dev = -1;
  XP_TRY(hipGetDevice(&dev), "current device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(XPRESS_ERR_HIP, "device %d outside the %d devices the static scratch supports", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    XP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "static scratch address");
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(XPRESS_ERR_HIP, "static scratch address %p is not 256-byte aligned", p);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return XPRESS_OK;
}

}  // namespace

extern "C" {

const char* xpress_last_error(void) { return g_err.c_str(); }

xpress_status xpress_workspace_size(int32_t n_max, int32_t B, int32_t r, int64_t V, int32_t C,
                                    int32_t k_max, size_t* bytes) {
  if (bytes == nullptr) return fail(XPRESS_ERR_ARG, "bytes is NULL");
  if (n_max < 0 || C < 0 || k_max < 0) return fail(XPRESS_ERR_ARG, "negative n_max, C or k_max");
  xpress_status st = check_dims(B, r, V);
  if (st != XPRESS_OK) return st;
  // every region grows with N, except the latent scratch, whose table-path part peaks where the
  // slices widen from 32 to 64 units and where the path stops (some N <= kTableMaxWorkgroups,
  // depending on M): the largest layout of any N <= n_max is at n_max or at one of those N
  size_t t = step_layout(n_max, B, r, kMaxH, V, C, k_max).total;
  for (int n = 1; n <= kTableMaxWorkgroups && n < n_max; ++n) {
    const size_t u = step_layout(n, B, r, kMaxH, V, C, k_max).total;
    t = u > t ? u : t;
  }
  *bytes = t;
  return XPRESS_OK;
}

xpress_status xpress_fold_mixer(const xpress_bf16* raw, int32_t r, int32_t B, xpress_bf16* mix_L,
                                xpress_stream stream) {
  xpress_status st = check_dims(B, r, 1);
  if (st != XPRESS_OK) return st;
  if (raw == nullptr || mix_L == nullptr) return fail(XPRESS_ERR_ARG, "raw or mix_L is NULL");
  if (raw == mix_L) return fail(XPRESS_ERR_ARG, "mix_L must not alias raw");
  XP_TRY(xpress::launch_fold_mixer(raw, r, B, mix_L, reinterpret_cast<hipStream_t>(stream)),
         "fold mixer");
  return XPRESS_OK;
}

xpress_status xpress_fold_embedding(const xpress_weights* w, float* w1p, xpress_stream stream) {
  if (w == nullptr) return fail(XPRESS_ERR_ARG, "weights struct is NULL");
  xpress_status st = check_dims(2, w->r, w->V);
  if (st != XPRESS_OK) return st;
  XP_PTR(w->w1);
  XP_PTR(w->in_proj);
  XP_PTR(w1p);
  XP_TRY(xpress::launch_fold_embedding(w->w1, w->in_proj, w->r, w->V, w1p,
                                       reinterpret_cast<hipStream_t>(stream)),
         "fold embedding");
  return XPRESS_OK;
}

xpress_status xpress_hidden_cache(const xpress_weights* w, const xpress_bf16* h, int32_t N,
                                  float* xh, void* ws, size_t ws_bytes, xpress_stream stream) {
  xpress_status st = check_weights(w, true, false, false);
  if (st != XPRESS_OK) return st;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (N == 0) return XPRESS_OK;
  XP_PTR(h);
  XP_PTR(xh);
  XP_PTR(ws);
  const size_t need = xpress::hidden_scratch_bytes(N * w->B, w->H, w->r);
  if (ws_bytes < need)
    return fail(XPRESS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for N=%d", ws_bytes, need, N);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* hdg = static_cast<float*>(ws);
  XP_TRY(xpress::launch_hidden_gemm(h, w->down_h, w->down_g, N * w->B, w->H, w->r, hdg, s), "hidden gemm");
  XP_TRY(xpress::launch_hidden_project(hdg, w->H, w->in_proj, N, w->B, w->r, xh, s), "hidden project");
  return XPRESS_OK;
}

xpress_status xpress_initial_block(const xpress_bf16* base, int64_t base_ld, const int64_t* anchor,
                                   int32_t N, int32_t B, int64_t V, int64_t* blk,
                                   xpress_stream stream) {
  xpress_status st = check_dims(B, 64, V);
  if (st != XPRESS_OK) return st;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (N == 0) return XPRESS_OK;
  st = check_base(base, base_ld, V);
  if (st != XPRESS_OK) return st;
  XP_PTR(anchor);
  XP_PTR(blk);
  XP_TRY(xpress::launch_initial_block(base, base_ld, anchor, N, B, V, blk,
                                      reinterpret_cast<hipStream_t>(stream)),
         "initial block");
  return XPRESS_OK;
}

xpress_status xpress_latent_pass(const xpress_weights* w, const int64_t* blk, const int64_t* am1,
                                 const float* xh, int32_t N, xpress_bf16* lat,
                                 uint32_t lat_layout, void* ws, size_t ws_bytes,
                                 xpress_stream stream) {
  xpress_status st = check_weights(w, false, true, false);
  if (st != XPRESS_OK) return st;
  st = check_layout(lat_layout);
  if (st != XPRESS_OK) return st;
  const bool frag = lat_layout == XPRESS_LAT_FRAGMENTS;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (N == 0) return XPRESS_OK;
  XP_PTR(blk);
  XP_PTR(am1);
  XP_PTR(xh);
  XP_PTR(lat);
  XP_PTR(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (use_table(w, N)) {
    const size_t need = xpress::latent_fused_scratch_bytes(N, w->r, w->M);
    if (ws_bytes < need)
      return fail(XPRESS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for N=%d", ws_bytes, need, N);
    XP_TRY(xpress::launch_latent_fused(nullptr, 0, const_cast<int64_t*>(blk), am1, xh, w->w1p,
                                       w->mix_L, w->w_gate, w->w_up, w->w_down, N, w->B, w->r,
                                       w->M, w->V, lat, static_cast<float*>(ws), nullptr, 0, s,
                                       true, frag),
           "latent");
    return XPRESS_OK;
  }
  const size_t need = xpress::latent_scratch_bytes(N, w->r, w->M);
  if (ws_bytes < need)
    return fail(XPRESS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for N=%d", ws_bytes, need, N);
  XP_TRY(xpress::launch_latent(nullptr, 0, const_cast<int64_t*>(blk), am1, xh, w->w1, w->in_proj,
                               w->mix_L, w->w_gate, w->w_up, w->w_down, N, w->B, w->r, w->M, w->V,
                               lat, ws, nullptr, 0, s, frag),
         "latent");
  return XPRESS_OK;
}

xpress_status xpress_readout_argmax(const xpress_weights* w, const xpress_bf16* lat,
                                    uint32_t lat_layout, const xpress_bf16* base,
                                    int64_t base_ld, int32_t N, int64_t* blk, int32_t* changed,
                                    void* ws, size_t ws_bytes, xpress_stream stream) {
  xpress_status st = check_weights(w, false, false, true);
  if (st != XPRESS_OK) return st;
  st = check_layout(lat_layout);
  if (st != XPRESS_OK) return st;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (N == 0) return XPRESS_OK;
  st = check_base(base, base_ld, w->V);
  if (st != XPRESS_OK) return st;
  XP_PTR(lat);
  XP_PTR(blk);
  XP_PTR(ws);
  const int rows = N * (w->B - 1);
  const int ntiles = xpress::readout_tiles(w->V, rows);
  const size_t need = (size_t)rows * ntiles * sizeof(uint2);
  if (ws_bytes < need)
    return fail(XPRESS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for N=%d", ws_bytes, need, N);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint2* part = static_cast<uint2*>(ws);
  XP_TRY(xpress::launch_readout_partial(lat, w->w2, base, base_ld, rows, w->V, w->r, part, nullptr, 0, s,
                                        lat_layout == XPRESS_LAT_FRAGMENTS),
         "readout");
  XP_TRY(xpress::launch_argmax_reduce(part, ntiles, rows, w->B, blk, changed, nullptr, 0, s),
         "argmax reduce");
  return XPRESS_OK;
}

xpress_status xpress_readout_tiles(int64_t V, int32_t rows, int32_t* ntiles) {
  if (ntiles == nullptr) return fail(XPRESS_ERR_ARG, "ntiles is NULL");
  xpress_status st = check_dims(2, 64, V);
  if (st != XPRESS_OK) return st;
  if (rows < 1) return fail(XPRESS_ERR_ARG, "rows=%d < 1", rows);
  *ntiles = xpress::readout_tiles(V, rows);
  return XPRESS_OK;
}

xpress_status xpress_readout_partials(const xpress_weights* w, const xpress_bf16* lat,
                                      uint32_t lat_layout, const xpress_bf16* base,
                                      int64_t base_ld, int32_t N, uint32_t* part,
                                      xpress_stream stream) {
  xpress_status st = check_weights(w, false, false, true);
  if (st != XPRESS_OK) return st;
  st = check_layout(lat_layout);
  if (st != XPRESS_OK) return st;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (N == 0) return XPRESS_OK;
  st = check_base(base, base_ld, w->V);
  if (st != XPRESS_OK) return st;
  XP_PTR(lat);
  XP_PTR(part);
  XP_TRY(xpress::launch_readout_partial(lat, w->w2, base, base_ld, N * (w->B - 1), w->V, w->r,
                                        reinterpret_cast<uint2*>(part), nullptr, 0,
                                        reinterpret_cast<hipStream_t>(stream),
                                        lat_layout == XPRESS_LAT_FRAGMENTS),
         "readout");
  return XPRESS_OK;
}

xpress_status xpress_argmax_reduce(const uint32_t* part, int32_t ntiles, int32_t N, int32_t B,
                                   int64_t* blk, int32_t* changed, xpress_stream stream) {
  if (B < 2 || B > 16) return fail(XPRESS_ERR_ARG, "B=%d outside [2, 16]", B);
  if (N < 0 || ntiles < 1) return fail(XPRESS_ERR_ARG, "N=%d < 0 or ntiles=%d < 1", N, ntiles);
  if (N == 0) return XPRESS_OK;
  XP_PTR(part);
  XP_PTR(blk);
  XP_TRY(xpress::launch_argmax_reduce(reinterpret_cast<const uint2*>(part), ntiles, N * (B - 1), B,
                                      blk, changed, nullptr, 0,
                                      reinterpret_cast<hipStream_t>(stream)),
         "argmax reduce");
  return XPRESS_OK;
}

xpress_status xpress_topc_prepare(const xpress_weights* w, const xpress_bf16* base,
                                  int64_t base_ld, int32_t N, int32_t C, int64_t* cand,
                                  xpress_bf16* base_c, xpress_bf16* w2c, void* ws,
                                  size_t ws_bytes, xpress_stream stream) {
  xpress_status st = check_weights(w, false, false, true);
  if (st != XPRESS_OK) return st;
  if (N < 0) return fail(XPRESS_ERR_ARG, "N=%d < 0", N);
  if (C < 1) return fail(XPRESS_ERR_ARG, "C=%d < 1", C);
  if (N == 0) return XPRESS_OK;
  st = check_base(base, base_ld, w->V);
  if (st != XPRESS_OK) return st;
  XP_PTR(cand);
  XP_PTR(base_c);
  if (w2c != nullptr && (reinterpret_cast<uintptr_t>(w2c) & 15) != 0)
    return fail(XPRESS_ERR_ARG, "w2c is not 16-byte aligned");
  const int c = (int)(C < w->V ? C : w->V);
  const int rows = N * (w->B - 1);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the workspace, when it is large enough (and aligned), holds the selection's chunk maxima
  const bool ws_ok = ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 15) == 0 &&
                     ws_bytes >= xpress::topc_select_scratch_bytes(rows, w->V);
  XP_TRY(xpress::launch_topc_select(base, base_ld, rows, w->V, c, cand, base_c, nullptr, nullptr, 0,
                                    ws_ok ? static_cast<uint16_t*>(ws) : nullptr, s),
         "top-C select");
  if (w2c != nullptr)
    XP_TRY(xpress::launch_topc_gather(cand, w->w2, rows, c, w->r, w2c, s), "top-C gather");
  return XPRESS_OK;
}

xpress_status xpress_readout_argmax_topc(const xpress_bf16* lat, const xpress_bf16* w2c,
                                         const xpress_bf16* base_c, const int64_t* cand,
                                         int32_t N, int32_t B, int32_t r, int32_t c,
                                         int64_t* blk, int32_t* changed, xpress_stream stream) {
  xpress_status st = check_dims(B, r, 1);
  if (st != XPRESS_OK) return st;
  if (N < 0 || c < 1) return fail(XPRESS_ERR_ARG, "N=%d < 0 or c=%d < 1", N, c);
  if (N == 0) return XPRESS_OK;
  XP_PTR(lat);
  XP_PTR(w2c);
  if (base_c == nullptr || cand == nullptr || blk == nullptr)
    return fail(XPRESS_ERR_ARG, "base_c, cand or blk is NULL");
  XP_TRY(xpress::launch_topc_readout(lat, nullptr, 0, w2c, false, base_c, cand, N * (B - 1), B, r,
                                     c, blk, changed, nullptr, 0,
                                     reinterpret_cast<hipStream_t>(stream)),
         "top-C readout");
  return XPRESS_OK;
}

xpress_status xpress_readout_argmax_topc_ids(const xpress_weights* w, const xpress_bf16* lat,
                                             const xpress_bf16* base_c, const int64_t* cand,
                                             int32_t N, int32_t c, int64_t* blk, int32_t* changed,
                                             xpress_stream stream) {
  xpress_status st = check_weights(w, false, false, true);
  if (st != XPRESS_OK) return st;
  if (N < 0 || c < 1 || c > w->V)
    return fail(XPRESS_ERR_ARG, "N=%d < 0 or c=%d outside [1, V=%lld]", N, c, (long long)w->V);
  if (N == 0) return XPRESS_OK;
  XP_PTR(lat);
  if (base_c == nullptr || cand == nullptr || blk == nullptr)
    return fail(XPRESS_ERR_ARG, "base_c, cand or blk is NULL");
  XP_TRY(xpress::launch_topc_readout(lat, nullptr, 0, w->w2, true, base_c, cand, N * (w->B - 1),
                                     w->B, w->r, c, blk, changed, nullptr, 0,
                                     reinterpret_cast<hipStream_t>(stream)),
         "top-C readout");
  return XPRESS_OK;
}

xpress_status xpress_jacobi_step(const xpress_weights* w, const xpress_bf16* h,
                                 const xpress_bf16* base, int64_t base_ld, const int64_t* anchor,
                                 const int64_t* am1, int32_t N, int32_t K, int32_t C,
                                 uint32_t flags, int64_t* blk, int32_t* passes_run, void* ws,
                                 size_t ws_bytes, xpress_stream stream) {
  xpress_status st = check_weights(w, true, true, true);
  if (st != XPRESS_OK) return st;
  if (N < 0 || K < 0 || C < 0) return fail(XPRESS_ERR_ARG, "negative N, K or C");
  if (flags & ~(uint32_t)(XPRESS_INIT_FROM_BASE | XPRESS_STOP_AT_FIXED_POINT))
    return fail(XPRESS_ERR_ARG, "unknown flag bits 0x%x", flags);
  if (N == 0) return XPRESS_OK;
  st = check_base(base, base_ld, w->V);
  if (st != XPRESS_OK) return st;
  XP_PTR(h);
  XP_PTR(anchor);
  XP_PTR(am1);
  XP_PTR(blk);
  XP_PTR(ws);
  const Layout L = step_layout(N, w->B, w->r, w->H, w->V, C, K);
  if (ws_bytes < L.total)
    return fail(XPRESS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for N=%d, C=%d, K=%d",
                ws_bytes, L.total, N, C, K);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = w->B, r = w->r, rows = N * (B - 1);
  const int64_t V = w->V;
  float* hdg = at<float>(ws, L.hdg);
  float* xh = at<float>(ws, L.xh);
  xpress_bf16* lat = at<xpress_bf16>(ws, L.lat);
  void* lscr = at<char>(ws, L.lscr);
  const int c = C > 0 ? (int)(C < V ? C : V) : 0;
  const bool init = (flags & XPRESS_INIT_FROM_BASE) != 0;
  // the starting block: with candidates, the selection writes it (the best candidate is the
  // row's argmax; the anchor too); without, one launch computes it beside the hidden GEMM
  int64_t* cand = at<int64_t>(ws, L.cand);
  xpress_bf16* base_c = at<xpress_bf16>(ws, L.base_c);
  // per-pass change flags of the device-side early exit, cleared by the step's first launch
  const bool stop = (flags & XPRESS_STOP_AT_FIXED_POINT) != 0;
  int32_t* pf = stop ? at<int32_t>(ws, L.flags) : nullptr;
  if (c > 0)  // the hidden GEMM beside the selection (which also writes the starting block)
    XP_TRY(xpress::launch_topc_start(h, w->down_h, w->down_g, N * B, w->H, r, hdg, base, base_ld,
                                     rows, V, c, cand, base_c, anchor, init ? blk : nullptr, B,
                                     at<uint16_t>(ws, L.cmax), s, pf, K + 1),
           "hidden gemm + top-C select");
  else if (init)
    XP_TRY(xpress::launch_step_start(h, w->down_h, w->down_g, N * B, w->H, r, hdg, base, base_ld,
                                     anchor, N, B, V, blk, s, pf, K + 1),
           "hidden gemm + starting block");
  else
    XP_TRY(xpress::launch_hidden_gemm(h, w->down_h, w->down_g, N * B, w->H, r, hdg, s), "hidden gemm");
  XP_TRY(xpress::launch_hidden_project(hdg, w->H, w->in_proj, N, B, r, xh, s), "hidden project");
  if (!init) XP_TRY(xpress::launch_set_anchor(anchor, N, B, blk, s), "set anchor");
  const bool fused = use_table(w, N);
  if (stop && c == 0 && !init) XP_TRY(xpress::launch_flags_reset(pf, K + 1, s), "flags reset");
  uint2* part = at<uint2>(ws, L.part);
  const int ntiles = xpress::readout_tiles(V, rows);
  // Full vocabulary: the argmax reduce of pass p-1 runs inside pass p's first latent kernel (each
  // block finishes its own rows); only the last pass's reduce is a launch of its own. lat is kept
  // in the readout's fragment order (coalesced loads of every workgroup's lat fragments).
  const bool lat_frag = c == 0;
  for (int p = 0; p < K; ++p) {
    const uint2* prev = (c == 0 && p > 0) ? part : nullptr;
    // with candidates, the top-C readout sums the table path's latent shares itself
    if (fused)
      XP_TRY(xpress::launch_latent_fused(prev, ntiles, blk, am1, xh, w->w1p, w->mix_L, w->w_gate,
                                         w->w_up, w->w_down, N, B, r, w->M, V, lat,
                                         static_cast<float*>(lscr), pf, p, s, c == 0, lat_frag),
             "latent");
    else
      XP_TRY(xpress::launch_latent(prev, ntiles, blk, am1, xh, w->w1, w->in_proj, w->mix_L,
                                   w->w_gate, w->w_up, w->w_down, N, B, r, w->M, V, lat, lscr, pf,
                                   p, s, lat_frag),
             "latent");
    if (c > 0) {
      XP_TRY(xpress::launch_topc_readout(lat, fused ? static_cast<const float*>(lscr) : nullptr,
                                         xpress::share_slices(N, w->M), w->w2, true, base_c, cand, rows, B, r, c, blk,
                                         nullptr, pf, p, s),
             "top-C readout");
    } else {
      XP_TRY(xpress::launch_readout_partial(lat, w->w2, base, base_ld, rows, V, r, part, pf, p, s,
                                            lat_frag),
             "readout");
    }
  }
  // the last pass's reduce also writes the pass count; otherwise a launch of its own does
  const bool last_reduce = c == 0 && K > 0;
  if (last_reduce)
    XP_TRY(xpress::launch_argmax_reduce(part, ntiles, rows, B, blk, nullptr, pf, K - 1, s,
                                        passes_run),
           "argmax reduce");
  if (passes_run && !last_reduce)
    XP_TRY(xpress::launch_count_passes(pf, K, stop ? 1 : 0, passes_run, s), "count passes");
  return XPRESS_OK;
}

xpress_status xpress_jacobi_step_noalloc(const xpress_weights* w, const xpress_bf16* h,
                                         const xpress_bf16* base, int64_t base_ld,
                                         const int64_t* anchor, const int64_t* am1, int32_t N,
                                         int32_t K, int32_t C, uint32_t flags, int64_t* blk,
                                         int32_t* passes_run, xpress_stream stream) {
  if (w == nullptr) return fail(XPRESS_ERR_ARG, "weights struct is NULL");
  xpress_status st = check_dims(w->B, w->r, w->V);
  if (st != XPRESS_OK) return st;
  if (N < 0 || K < 0 || C < 0) return fail(XPRESS_ERR_ARG, "negative N, K or C");
  if (N == 0) return XPRESS_OK;
  const size_t need = step_layout(N, w->B, w->r, w->H, w->V, C, K).total;
  if (need > kStaticScratchBytes)
    return fail(XPRESS_ERR_WORKSPACE,
                "the step needs %zu bytes of scratch (N=%d, C=%d, K=%d), more than the %zu bytes "
                "of the allocation-free step's static scratch; use xpress_jacobi_step with a "
                "caller workspace", need, N, C, K, kStaticScratchBytes);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != XPRESS_OK) return st;
  return xpress_jacobi_step(w, h, base, base_ld, anchor, am1, N, K, C, flags, blk, passes_run, ws,
                            kStaticScratchBytes, stream);
}

xpress_status xpress_jacobi_step_graph(const xpress_weights* w, const xpress_bf16* h,
                                       const xpress_bf16* base, int64_t base_ld,
                                       const int64_t* anchor, const int64_t* am1, int32_t N,
                                       int32_t K, int32_t C, uint32_t flags, int64_t* blk,
                                       int32_t* passes_run, void* ws, size_t ws_bytes,
                                       void** graph) {
  XP_PTR(graph);
  *graph = nullptr;
  hipStream_t cs = nullptr;
  XP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "capture stream");
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(XPRESS_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
  }
  const xpress_status st = xpress_jacobi_step(w, h, base, base_ld, anchor, am1, N, K, C, flags,
                                              blk, passes_run, ws, ws_bytes,
                                              reinterpret_cast<xpress_stream>(cs));
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (st != XPRESS_OK) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return fail(XPRESS_ERR_HIP, "end capture: %s", hipGetErrorString(e));
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(XPRESS_ERR_HIP, "instantiate: %s", hipGetErrorString(e));
  *graph = ge;
  return XPRESS_OK;
}

xpress_status xpress_graph_launch(void* graph, xpress_stream stream) {
  XP_PTR(graph);
  XP_TRY(hipGraphLaunch(reinterpret_cast<hipGraphExec_t>(graph),
                        reinterpret_cast<hipStream_t>(stream)),
         "graph launch");
  return XPRESS_OK;
}

xpress_status xpress_graph_destroy(void* graph) {
  if (!graph) return XPRESS_OK;
  XP_TRY(hipGraphExecDestroy(reinterpret_cast<hipGraphExec_t>(graph)), "graph destroy");
  return XPRESS_OK;
}

}  // extern "C"
