/*
 * xpress.h -- C ABI of the MI355X (gfx950) XPress Jacobi block-refiner pass library.
 *
 * The XPress refiner drafts a block of B tokens per request: slot 0 holds the verified anchor and
 * slots 1..B-1 hold draft tokens. One Jacobi pass re-derives every draft slot from the block as it
 * stood at the start of the pass (definitions: vLLM API pages "vllm.model_executor.models.
 * qwen3_xpress", class XPressRefinerHead, and "vllm.v1.worker.gpu.spec_decode.xpress.kernels",
 * module docstring):
 *   latent  x[b] = xh[b] + P_e . w1[prev[b]],  prev[0] = am1, prev[b] = blk[b-1]
 *           u[b] = sum_{j<=b} L[:, b, j] * x[j]               (per-channel causal mixer)
 *           lat[b] = u[b] + w_down . (silu(w_gate . u[b]) * (w_up . u[b]))     (b >= 1)
 *   readout logit[b, v] = base[b, v] + lat[b] . w2[v]
 *   argmax  blk[b] = argmax_v logit[b, v]   (ties: lowest vocabulary id)
 * with xh the pass-invariant hidden cache (in_proj's hidden half applied to
 * [down_h(h) ++ down_g(mean_b h)]). With top-C the readout only scores the C candidates taken
 * once per step from the base logits.
 *
 * Conventions shared by every call:
 *   - Every pointer is a DEVICE pointer owned by the caller, except the xpress_weights struct
 *     itself (host memory, read during the call only) and out-parameters named *_bytes (host).
 *   - bf16 tensors are passed as their 16-bit patterns (xpress_bf16). Token ids are int64.
 *   - Layouts are dense row-major with the shapes given, except base logits, which take a row
 *     stride (elements) base_ld >= V, a multiple of 8; the base buffer must be readable for
 *     rows * base_ld elements (the last row too is padded to the full stride): kernels read whole
 *     8-element groups up to the padded row end and ignore the ids >= V.
 *   - Rows of the readout: row p = n*(B-1) + (b-1) is slot b (1..B-1) of block n.
 *   - Every call only enqueues work on `stream` (NULL = the null stream) and returns; none
 *     allocates, frees or synchronises, so a sequence of calls can be captured into a HIP graph.
 *   - Argument errors are detected on the host before anything is enqueued; the call then returns
 *     a non-zero status and xpress_last_error() describes it. XPRESS_ERR_HIP reports a launch
 *     failure from the HIP runtime.
 *   - N == 0 is a no-op that returns XPRESS_OK.
 *   - Supported shapes on the GPU path: r in {64, 128, 256}; 2 <= B <= 16; M in
 *     {64, 128, 256, 512, 1024}; H a multiple of 64 in [64, 16384]; V >= 1 and V*r < 2^31; all
 *     pointers 16-byte aligned and base_ld a multiple of 8 elements, V <= base_ld <= 2^27.
 *     Other values are XPRESS_ERR_ARG.
 *   - Capacity: a workspace sized by xpress_workspace_size(n_max, ...) serves every N <= n_max;
 *     a call whose N needs more than ws_bytes (N beyond the n_max the workspace was sized for,
 *     among other cases) returns XPRESS_ERR_WORKSPACE before enqueueing anything. That one
 *     status covers both the capacity and the size check, since the size in bytes is what
 *     records n_max.
 *   - Inputs should be finite. For -inf/NaN values the chosen tokens are unspecified (except
 *     that -inf orders below every finite value and ties like any other value), but every id
 *     written is in [0, V) (for top-C: one of the row's candidates).
 */
#ifndef XPRESS_H
#define XPRESS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t xpress_bf16;             /* bfloat16 bit pattern */
typedef struct ihipStream_t* xpress_stream; /* hipStream_t */

typedef enum {
  XPRESS_OK = 0,
  XPRESS_ERR_ARG = 1,       /* null/misaligned pointer, unsupported shape, C > V, K < 0, ... */
  XPRESS_ERR_WORKSPACE = 2, /* the workspace is smaller than the call needs for this N */
  XPRESS_ERR_HIP = 3        /* the HIP runtime reported an error at launch */
} xpress_status;

/* Parameters of one refiner head (qwen3_xpress page, XPressRefinerHead constructor), in the
 * nn.Linear layout [out_features, in_features]. Device pointers, bf16. */
typedef struct {
  int32_t B; /* slots per block, anchor included */
  int32_t r; /* latent rank */
  int32_t H; /* model hidden size */
  int32_t M; /* SwiGLU hidden size (mlp_hidden) */
  int64_t V; /* vocabulary size */
  const xpress_bf16* w1;      /* [V, r]   token embedding                                      */
  const xpress_bf16* down_h;  /* [r, H]   per-slot hidden projection                           */
  const xpress_bf16* down_g;  /* [r, H]   projection of the block-mean hidden state            */
  const xpress_bf16* in_proj; /* [r, 3r]  columns [0,r) act on down_h, [r,2r) on down_g,
                                          [2r,3r) on the token embedding                       */
  const xpress_bf16* mix_L;   /* [B, B, r] FOLDED mixer, channel innermost (the layout of the
                                           kernels page's latent kernel):
                                           mix_L[(b*B + j)*r + c] = raw[c,b,j]*[j<=b] + [j==b]
                                           (qwen3_xpress page, fold_from_raw_); only j <= b is
                                           read                                                */
  const xpress_bf16* w_gate;  /* [M, r]                                                        */
  const xpress_bf16* w_up;    /* [M, r]                                                        */
  const xpress_bf16* w_down;  /* [r, M]                                                        */
  const xpress_bf16* w2;      /* [V, r]   readout                                              */
  const float* w1p;           /* [V, r]   OPTIONAL (NULL: not used), fp32: the embedding table with
                                          in_proj's embedding block applied,
                                          w1p[v, c] = sum_k in_proj[c, 2r+k] * w1[v, k]
                                          (xpress_fold_embedding). When given and
                                          N * M/64 <= 448 (one workgroup per block and 64-unit
                                          slice, two per CU in one round: N <= 56 at M = 512),
                                          the latent stage gathers its rows instead of
                                          projecting w1's rows every pass and runs as two
                                          launches instead of three (beyond that the
                                          three-kernel path is faster and is used); results
                                          agree with the NULL path within fp32 rounding        */
} xpress_weights;

/* Layouts of the latent rows lat (N*(B-1) readout rows of r channels, bf16):
 *   XPRESS_LAT_ROWS       row-major [N*(B-1), r];
 *   XPRESS_LAT_FRAGMENTS  the order in which the full-vocabulary readout's matrix core takes them
 *                         (the layout a draft step keeps): rows in tiles of 32; for tile T,
 *                         16-channel group s and lane l = 32*h + (p % 32), the 8 channels
 *                         16*s + 8*h .. +7 of row p = 32*T + (p % 32) are the 16 bytes at byte
 *                         offset ((T*(r/16) + s)*64 + l)*16. The buffer holds ceil(N*(B-1)/32)
 *                         whole tiles (the rows past N*(B-1) are never written or used). */
#define XPRESS_LAT_ROWS 0u
#define XPRESS_LAT_FRAGMENTS 1u

/* Flags of xpress_jacobi_step. */
#define XPRESS_INIT_FROM_BASE 1u      /* blk[:,0] = anchor, blk[:,1:] = argmax(base) first    */
#define XPRESS_STOP_AT_FIXED_POINT 2u /* passes after the first pass that changes no slot
                                          return at once on the device (K stays the launch
                                          count, so the step remains graph-capturable)        */

/* Bytes of device workspace the calls below need for up to n_max blocks, C candidates (0 = full
 * vocabulary) and up to k_max passes per step. Allocate once; any call with N <= n_max, the same
 * B, r, V, C and K <= k_max fits. Returns XPRESS_ERR_ARG for an unsupported shape. */
xpress_status xpress_workspace_size(int32_t n_max, int32_t B, int32_t r, int64_t V, int32_t C,
                                    int32_t k_max, size_t* bytes);

/* Fold of a raw (training-form) mixer into its serving form (qwen3_xpress page,
 * XPressRefinerHead.fold_from_raw_): L[c,b,j] = raw[c,b,j] * [j <= b] + [j == b], computed in
 * fp32 and rounded to bf16 (round to nearest even), as copying into a bf16 parameter does, and
 * stored channel innermost: mix_L[(b*B + j)*r + c] = L[c,b,j].
 * raw: [r, B, B] bf16 (the parameter's own layout); mix_L: [B, B, r] bf16 (written; must not
 * alias raw). */
xpress_status xpress_fold_mixer(const xpress_bf16* raw, int32_t r, int32_t B, xpress_bf16* mix_L,
                                xpress_stream stream);

/* Projected embedding table (the embedding block of in_proj that qwen3_xpress page,
 * jacobi_refine_greedy, applies to the gathered token embeddings every pass, applied here once
 * to every row of w1): w1p[v, c] = sum_k in_proj[c, 2r + k] * w1[v, k] for v < V, c < r, with
 * bf16 operands and fp32 accumulation. Reads w->w1, w->in_proj, w->r, w->V (w->w1p is ignored).
 * w1p: [V, r] fp32 (written, caller-owned, 16-byte aligned; 4*V*r bytes). Pass it as
 * xpress_weights.w1p afterwards; recompute it whenever w1 or in_proj change. */
xpress_status xpress_fold_embedding(const xpress_weights* w, float* w1p, xpress_stream stream);

/* Hidden cache (qwen3_xpress page, hidden_cache, and the hidden half of in_proj that
 * jacobi_refine_greedy applies once per step):
 *   xh[n,b,:] = in_proj[:, 0:r] . (down_h . h[n,b]) + in_proj[:, r:2r] . (down_g . mean_b h[n,b])
 * h: [N, B, H] bf16. xh: [N, B, r] fp32 (written). ws: workspace of ws_bytes bytes. */
xpress_status xpress_hidden_cache(const xpress_weights* w, const xpress_bf16* h, int32_t N,
                                  float* xh, void* ws, size_t ws_bytes, xpress_stream stream);

/* Starting block of a step (qwen3_xpress page, jacobi_refine_greedy): blk[n,0] = anchor[n] and
 * blk[n,b] = argmax_v base[n*(B-1)+b-1, v] for b >= 1 (lowest id on ties).
 * base: [N*(B-1), V] bf16, row stride base_ld. anchor: [N]. blk: [N, B] (written). */
xpress_status xpress_initial_block(const xpress_bf16* base, int64_t base_ld,
                                   const int64_t* anchor, int32_t N, int32_t B, int64_t V,
                                   int64_t* blk, xpress_stream stream);

/* Latent stage of one pass (kernels page, _xpress_latent_kernel; qwen3_xpress page,
 * _refine_latent): reads blk, never writes it. Token ids outside [0, V) contribute a zero
 * embedding.
 * blk: [N, B]; am1: [N] (token before each anchor); xh: [N, B, r] fp32 from xpress_hidden_cache;
 * lat: [N, B-1, r] bf16 (written; row n*(B-1)+b-1 is slot b) in lat_layout (XPRESS_LAT_ROWS or
 * XPRESS_LAT_FRAGMENTS; other values are XPRESS_ERR_ARG). ws: scratch of ws_bytes bytes (a
 * workspace sized by xpress_workspace_size for at least N blocks is enough). */
xpress_status xpress_latent_pass(const xpress_weights* w, const int64_t* blk, const int64_t* am1,
                                 const float* xh, int32_t N, xpress_bf16* lat,
                                 uint32_t lat_layout, void* ws, size_t ws_bytes,
                                 xpress_stream stream);

/* Full-vocabulary readout and argmax (kernels page, fused_add_argmax_to_blk; qwen3_xpress page,
 * refine_bias): blk[n, b] = argmax_v (base[p, v] + lat[p] . w2[v]) for p = n*(B-1)+b-1, written in
 * place for slots 1..B-1. The [N*(B-1), V] logits are never stored.
 * lat: [N*(B-1), r] bf16 in lat_layout; base: [N*(B-1), V] bf16 stride base_ld; blk: [N, B]
 * in/out. changed (nullable): set to 1 if any slot took a new value (never cleared by this
 * call). */
xpress_status xpress_readout_argmax(const xpress_weights* w, const xpress_bf16* lat,
                                    uint32_t lat_layout, const xpress_bf16* base,
                                    int64_t base_ld, int32_t N, int64_t* blk, int32_t* changed,
                                    void* ws, size_t ws_bytes, xpress_stream stream);

/* The two stages of xpress_readout_argmax, for callers that reduce the per-range winners
 * themselves (for example across GPUs that each hold a slice of the vocabulary) and for timing
 * the readout GEMM on its own (kernels page, _xpress_add_argmax_partial_kernel and
 * _xpress_add_argmax_reduce_to_blk_kernel).
 * xpress_readout_tiles: number of partials per readout row for `rows` = N*(B-1) readout rows:
 *   the vocabulary is cut into ntiles contiguous ranges of whole 32-id steps, ntiles =
 *   min(ceil(V / 32), 256) up to 512 rows and min(ceil(V / 32), max(8, floor(256 / k) rounded
 *   down to a multiple of 8)) with k = ceil(rows / 512) beyond (about one workgroup per CU).
 *   With S = ceil(V / 32) steps, range t holds the ids of steps floor(S*t / ntiles) up to (not
 *   including) floor(S*(t+1) / ntiles), the last clipped to V. rows < 1 is XPRESS_ERR_ARG.
 * xpress_readout_partials: part[t * N*(B-1) + p] = {bits of the fp32 maximum of base + lat . w2
 *   over range t of row p, the lowest vocabulary id attaining it}. part: [ntiles, N*(B-1)] pairs
 *   of uint32, range-major (caller-owned, 8 bytes each). lat in lat_layout.
 * xpress_argmax_reduce: blk[n, b] = the id of the largest pair of row p = n*(B-1)+b-1 (ties:
 *   lowest id), written in place; `changed` as in xpress_readout_argmax. */
xpress_status xpress_readout_tiles(int64_t V, int32_t rows, int32_t* ntiles);
xpress_status xpress_readout_partials(const xpress_weights* w, const xpress_bf16* lat,
                                      uint32_t lat_layout, const xpress_bf16* base,
                                      int64_t base_ld, int32_t N, uint32_t* part,
                                      xpress_stream stream);
xpress_status xpress_argmax_reduce(const uint32_t* part, int32_t ntiles, int32_t N, int32_t B,
                                   int64_t* blk, int32_t* changed, xpress_stream stream);

/* Top-C preparation, once per step (qwen3_xpress page, top-C branch of jacobi_refine_greedy):
 * cand[p] = the c = min(C, V) ids with the largest base[p, :] under the order (value descending,
 * id ascending), stored in ascending id order; base_c[p, k] = base[p, cand[p, k]];
 * w2c[p, k, :] = w2[cand[p, k], :] (the gather is skipped when w2c is NULL, for callers of
 * xpress_readout_argmax_topc_ids, which reads the rows from w2 through cand).
 * cand: [N*(B-1), c] int64; base_c: [N*(B-1), c] bf16; w2c: [N*(B-1), c, r] bf16 (written;
 * nullable, else 16-byte aligned).
 * ws (optional, may be NULL): device scratch for rows of more than 153,600 ids (rows up to that
 * length keep the selection's per-chunk maxima in LDS and ignore ws). For rows of 153,601 to
 * 524,288 ids, when ws is 16-byte aligned and holds at least N*(B-1) * 8*ceil(ceil(V/8)/8) * 2
 * bytes, the selection keeps per-chunk maxima there and its second pass over base reads only the
 * chunks that can hold an answer; otherwise (and for longer rows) it reads base three times. The
 * result is the same either way. xpress_jacobi_step's workspace includes this. */
xpress_status xpress_topc_prepare(const xpress_weights* w, const xpress_bf16* base,
                                  int64_t base_ld, int32_t N, int32_t C, int64_t* cand,
                                  xpress_bf16* base_c, xpress_bf16* w2c, void* ws,
                                  size_t ws_bytes, xpress_stream stream);

/* Top-C readout and argmax (kernels page, _xpress_topc_argmax_to_blk_kernel): for every row p,
 * k* = argmax_k (base_c[p, k] + lat[p] . w2c[p, k]) and blk[n, b] = cand[p, k*]; ties go to the
 * lowest vocabulary id cand[p, k], whatever the order of the candidates in the row (the
 * qwen3_xpress page notes that the candidate order does not matter). Shapes as in
 * xpress_topc_prepare with c candidates per row; cand may hold the ids in any order. */
xpress_status xpress_readout_argmax_topc(const xpress_bf16* lat, const xpress_bf16* w2c,
                                         const xpress_bf16* base_c, const int64_t* cand,
                                         int32_t N, int32_t B, int32_t r, int32_t c,
                                         int64_t* blk, int32_t* changed, xpress_stream stream);

/* The same top-C readout with the candidates' rows read from w->w2 through their ids (w2[cand[p,
 * k]] in place of w2c[p, k]; same result): no gathered copy is needed. This is the form a draft
 * step runs. Shapes and errors as in xpress_readout_argmax_topc; c in [1, w->V]; every
 * cand[p, k] must be in [0, w->V) (as xpress_topc_prepare writes them; not checked). */
xpress_status xpress_readout_argmax_topc_ids(const xpress_weights* w, const xpress_bf16* lat,
                                             const xpress_bf16* base_c, const int64_t* cand,
                                             int32_t N, int32_t c, int64_t* blk,
                                             int32_t* changed, xpress_stream stream);

/* One draft step (qwen3_xpress page, jacobi_refine_greedy): hidden cache, starting block (with
 * XPRESS_INIT_FROM_BASE; otherwise blk[:, 1:] is taken as given and blk[:, 0] is set to anchor),
 * top-C preparation when C > 0 (candidates and base_c; the passes read the candidates' w2 rows
 * through their ids, as xpress_readout_argmax_topc_ids), then K passes of latent + readout +
 * argmax. On return blk[:, 1:] is the draft.
 * h: [N, B, H]; base: [N*(B-1), V] stride base_ld; anchor, am1: [N]; blk: [N, B] in/out.
 * passes_run (nullable, device int32): number of passes that ran (with
 * XPRESS_STOP_AT_FIXED_POINT, the pass that changed nothing is counted). */
xpress_status xpress_jacobi_step(const xpress_weights* w, const xpress_bf16* h,
                                 const xpress_bf16* base, int64_t base_ld, const int64_t* anchor,
                                 const int64_t* am1, int32_t N, int32_t K, int32_t C,
                                 uint32_t flags, int64_t* blk, int32_t* passes_run, void* ws,
                                 size_t ws_bytes, xpress_stream stream);

/* The same draft step as xpress_jacobi_step, for callers that cannot allocate device memory or
 * hand over a workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no ws argument, and the call allocates nothing. Its scratch is a static array of
 * the library on each GPU (64 MiB, created with the library's code object on that GPU and held
 * until the process ends); the first call on a GPU looks up its address there. Every call on one
 * GPU shares that array, so calls that overlap on one GPU (concurrent streams or threads) race
 * and must be serialised by the caller; each call clears what it needs cleared itself, so
 * nothing carries over from the previous call. A step whose workspace (xpress_workspace_size for
 * its N, C and K) exceeds 64 MiB returns XPRESS_ERR_WORKSPACE before enqueueing anything: 64 MiB
 * covers a full-vocabulary or top-512 step of up to 256 blocks at B = 16, r = 256, V = 151936,
 * K = 15. Arguments, results and other errors as in
 * xpress_jacobi_step. */
xpress_status xpress_jacobi_step_noalloc(const xpress_weights* w, const xpress_bf16* h,
                                         const xpress_bf16* base, int64_t base_ld,
                                         const int64_t* anchor, const int64_t* am1, int32_t N,
                                         int32_t K, int32_t C, uint32_t flags, int64_t* blk,
                                         int32_t* passes_run, xpress_stream stream);

/* A draft step recorded once as a HIP graph and replayed with one launch (the pages capture
 * the pass loop in a graph with fixed buffer addresses: qwen3_xpress page, jacobi_refine_greedy;
 * kernels page, module docstring). xpress_jacobi_step_graph checks the arguments exactly as
 * xpress_jacobi_step does, then records that step's kernels on a private stream into a graph and
 * instantiates it; nothing runs. *graph receives an opaque handle. Every xpress_graph_launch
 * enqueues the whole step on `stream` with the recorded pointers and sizes, so the buffers must
 * stay allocated, and their contents are read at launch time (new h, base, anchor, am1 values are
 * picked up; blk is rewritten). With XPRESS_STOP_AT_FIXED_POINT the passes after convergence
 * exit on the device, as in the eager call. Creating a graph allocates host-side objects; the
 * launch allocates nothing. xpress_graph_destroy releases the handle (NULL is a no-op). Errors:
 * those of xpress_jacobi_step, XPRESS_ERR_HIP if recording or instantiation fails. */
xpress_status xpress_jacobi_step_graph(const xpress_weights* w, const xpress_bf16* h,
                                       const xpress_bf16* base, int64_t base_ld,
                                       const int64_t* anchor, const int64_t* am1, int32_t N,
                                       int32_t K, int32_t C, uint32_t flags, int64_t* blk,
                                       int32_t* passes_run, void* ws, size_t ws_bytes,
                                       void** graph);
xpress_status xpress_graph_launch(void* graph, xpress_stream stream);
xpress_status xpress_graph_destroy(void* graph);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char* xpress_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XPRESS_H */
