/*
 * xpress_oracle.c -- plain, slow CPU oracle of the XPress Jacobi block-refiner pass.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code, header, table or
 * helper with the HIP library; the only thing the two sides have in common is the seeded input
 * generator.
 *
 * What it follows (vLLM API documentation pages):
 *   [qwen3_xpress] "vllm.model_executor.models.qwen3_xpress", class XPressRefinerHead:
 *       fold_from_raw_, hidden_cache, _refine_latent, refine_bias, jacobi_refine_greedy.
 *   [kernels]      "vllm.v1.worker.gpu.spec_decode.xpress.kernels": the module docstring's
 *       four-stage pass definition and the docstrings of _xpress_latent_kernel,
 *       _xpress_add_argmax_partial_kernel / _reduce_to_blk_kernel and
 *       _xpress_topc_argmax_to_blk_kernel.
 *
 * Arithmetic: every input value arrives as float (bf16 values widened exactly, or fp32 draws);
 * every sum, product and comparison is done in double, in natural index order, one element at a
 * time. No blocking, no fusion, no reordering. OpenMP only splits independent outputs (rows of
 * the readout, blocks of the latent) between threads; no single sum is ever split, so the result
 * does not depend on the thread count.
 *
 * Readings where the pages leave a point open (each is also listed in the design notes):
 *   - argmax ties go to the lowest vocabulary id (torch.argmax returns the first maximum);
 *   - top-C selects by (value descending, id ascending) and returns the ids in ascending order;
 *     its argmax ties also go to the lowest vocabulary id, so the candidate order never matters;
 *   - the hidden-cache mean runs over all B slots, the anchor slot included;
 *   - the folded mixer is read only at j <= b (its upper triangle is zero after the fold);
 *   - slot 0's latent is formed (the mixer needs it) but it has no MLP output and no readout.
 *
 * Parity pins: every function here is pinned by tests that do not re-type its formula (closed
 * forms, special cases that reduce to a library routine, exact dyadic arithmetic, brute-force
 * sequential decoding); see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------ */
/* threads                                                                                     */

void xo_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int xo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Fold of the raw mixer into its serving form (qwen3_xpress, XPressRefinerHead.fold_from_raw_):
 * keep the lower triangle (j <= b) of each channel's B x B matrix and add the identity.
 * raw, L: [r, B, B], index [c][b][j].                                                          */
void xo_fold_mixer(const float* raw, int r, int B, double* L) {
  for (int c = 0; c < r; ++c)
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < B; ++j) {
        size_t o = ((size_t)c * B + b) * B + j;
        double v = (j <= b) ? (double)raw[o] : 0.0;
        if (j == b) v += 1.0;
        L[o] = v;
      }
}

/* ------------------------------------------------------------------------------------------ */
/* Pass-invariant hidden cache (qwen3_xpress, XPressRefinerHead.hidden_cache, and the hidden half
 * of in_proj that jacobi_refine_greedy applies once per step):
 *   g[n]     = mean over the B slots of h[n, b]             (dim 1 of [N, B, H])
 *   hd[n, b] = down_h . h[n, b]                              (down_h: [r, H])
 *   hg[n]    = down_g . g[n]                                 (down_g: [r, H])
 *   xh[n, b, i] = sum_k P[i, k] hd[n, b, k] + sum_k P[i, r + k] hg[n, k]    (P = in_proj [r, 3r])
 * h: [N, B, H]; xh: [N, B, r].                                                                 */
void xo_hidden_cache(const float* h, const float* down_h, const float* down_g,
                     const float* in_proj, int N, int B, int H, int r, double* xh) {
  double* g = (double*)malloc(sizeof(double) * (size_t)H);
  double* hd = (double*)malloc(sizeof(double) * (size_t)B * r);
  double* hg = (double*)malloc(sizeof(double) * (size_t)r);
  for (int n = 0; n < N; ++n) {
    for (int k = 0; k < H; ++k) {
      double s = 0.0;
      for (int b = 0; b < B; ++b) s += (double)h[((size_t)n * B + b) * H + k];
      g[k] = s / (double)B;
    }
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < r; ++i) {
        double s = 0.0;
        for (int k = 0; k < H; ++k)
          s += (double)down_h[(size_t)i * H + k] * (double)h[((size_t)n * B + b) * H + k];
        hd[(size_t)b * r + i] = s;
      }
    for (int i = 0; i < r; ++i) {
      double s = 0.0;
      for (int k = 0; k < H; ++k) s += (double)down_g[(size_t)i * H + k] * g[k];
      hg[i] = s;
    }
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < r; ++i) {
        double s = 0.0;
        for (int k = 0; k < r; ++k) s += (double)in_proj[(size_t)i * 3 * r + k] * hd[(size_t)b * r + k];
        for (int k = 0; k < r; ++k) s += (double)in_proj[(size_t)i * 3 * r + r + k] * hg[k];
        xh[((size_t)n * B + b) * r + i] = s;
      }
  }
  free(g);
  free(hd);
  free(hg);
}

/* ------------------------------------------------------------------------------------------ */
/* Argmax of one row of length n with stride 1 (double values). Ties go to the lowest index.
 * *gap = best - (largest value at any other index); 0 when the maximum occurs twice.          */
static int64_t argmax_with_gap(const double* v, int64_t n, double* gap) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  if (gap) {
    double second = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
      if (i != best && v[i] > second) second = v[i];
    *gap = (n > 1) ? v[best] - second : INFINITY;
  }
  return best;
}

/* Starting block of a step (qwen3_xpress, jacobi_refine_greedy): slot 0 holds the anchor and
 * slot b >= 1 the argmax of that slot's base logits. base: [N*(B-1), V] with row stride ld;
 * row n*(B-1) + b-1 is slot b of block n. blk: [N, B].                                         */
void xo_initial_block(const float* base, int64_t ld, const int64_t* anchor, int N, int B,
                      int64_t V, int64_t* blk) {
  for (int n = 0; n < N; ++n) {
    blk[(size_t)n * B] = anchor[n];
    for (int b = 1; b < B; ++b) {
      const float* row = base + ((int64_t)n * (B - 1) + (b - 1)) * ld;
      int64_t best = 0;
      for (int64_t v = 1; v < V; ++v)
        if ((double)row[v] > (double)row[best]) best = v;
      blk[(size_t)n * B + b] = best;
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Top-C candidate set (qwen3_xpress, jacobi_refine_greedy, top-C branch): per base row, the
 * c = min(C, V) ids with the largest base logits. The pages leave the rule at the boundary open;
 * this takes the total order (value descending, id ascending) and returns the selected ids in
 * ascending id order. base: [rows, V] stride ld; cand: [rows, c].                              */
typedef struct {
  double v;
  int64_t id;
} xo_key;

static int key_cmp(const void* a, const void* b) {
  const xo_key* x = (const xo_key*)a;
  const xo_key* y = (const xo_key*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int id_cmp(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x < y) ? -1 : (x > y);
}

void xo_topc_select(const float* base, int64_t ld, int64_t rows, int64_t V, int C, int64_t* cand) {
  int64_t c = (C < V) ? C : V;
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < rows; ++p) {
    xo_key* keys = (xo_key*)malloc(sizeof(xo_key) * (size_t)V);
    for (int64_t v = 0; v < V; ++v) {
      keys[v].v = (double)base[p * ld + v];
      keys[v].id = v;
    }
    qsort(keys, (size_t)V, sizeof(xo_key), key_cmp);
    int64_t* out = cand + p * c;
    for (int64_t k = 0; k < c; ++k) out[k] = keys[k].id;
    qsort(out, (size_t)c, sizeof(int64_t), id_cmp);
    free(keys);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Weights of the refiner head in nn.Linear layouts [out, in] (qwen3_xpress, constructor).      */
typedef struct {
  int B, r, M;
  int64_t V;
  const float* w1;      /* [V, r]   token embedding            */
  const float* in_proj; /* [r, 3r]  columns [2r, 3r) act on the embedding */
  const double* L;      /* [r, B, B] folded mixer              */
  const float* w_gate;  /* [M, r]                              */
  const float* w_up;    /* [M, r]                              */
  const float* w_down;  /* [r, M]                              */
} xo_latent_weights;

/* Latent of one block (qwen3_xpress, XPressRefinerHead._refine_latent, with the pass definition
 * of the kernels page): for every slot b,
 *   prev[0] = am1, prev[b] = blk[b-1]                      (slot b reads the previous slot's token)
 *   x[b, i] = xh[b, i] + sum_k P[i, 2r + k] * w1[prev[b], k]
 *   u[b, i] = sum_{j <= b} L[i, b, j] * x[j, i]             (per-channel causal mixer)
 * and for slots b >= 1 (slot 0 is never read out)
 *   a = w_gate . u[b],  c = w_up . u[b],  s_m = silu(a_m) * c_m,  silu(z) = z / (1 + e^-z)
 *   lat[b-1, i] = u[b, i] + sum_m w_down[i, m] * s_m.
 * blk_n: [B] tokens of this block; xh_n: [B, r]; lat_n: [B-1, r]; u_n: [B, r] or NULL.
 * Scratch x, u: [B, r]; a: [M].                                                               */
static void latent_block(const xo_latent_weights* w, const int64_t* blk_n, int64_t am1_n,
                         const double* xh_n, double* lat_n, double* u_out, double* x, double* u,
                         double* a) {
  const int B = w->B, r = w->r, M = w->M;
  for (int b = 0; b < B; ++b) {
    int64_t tok = (b == 0) ? am1_n : blk_n[b - 1];
    const float* e = w->w1 + tok * (int64_t)r;
    for (int i = 0; i < r; ++i) {
      double s = 0.0;
      for (int k = 0; k < r; ++k) s += (double)w->in_proj[(size_t)i * 3 * r + 2 * r + k] * (double)e[k];
      x[(size_t)b * r + i] = xh_n[(size_t)b * r + i] + s;
    }
  }
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < r; ++i) {
      double s = 0.0;
      for (int j = 0; j <= b; ++j) s += w->L[((size_t)i * B + b) * B + j] * x[(size_t)j * r + i];
      u[(size_t)b * r + i] = s;
    }
  if (u_out) memcpy(u_out, u, sizeof(double) * (size_t)B * r);
  for (int b = 1; b < B; ++b) {
    const double* ub = u + (size_t)b * r;
    for (int m = 0; m < M; ++m) {
      double sa = 0.0, sc = 0.0;
      for (int i = 0; i < r; ++i) sa += (double)w->w_gate[(size_t)m * r + i] * ub[i];
      for (int i = 0; i < r; ++i) sc += (double)w->w_up[(size_t)m * r + i] * ub[i];
      double silu = sa / (1.0 + exp(-sa));
      a[m] = silu * sc;
    }
    for (int i = 0; i < r; ++i) {
      double s = 0.0;
      for (int m = 0; m < M; ++m) s += (double)w->w_down[(size_t)i * M + m] * a[m];
      lat_n[(size_t)(b - 1) * r + i] = ub[i] + s;
    }
  }
}

/* Latent for N blocks. blk: [N, B]; am1: [N]; xh: [N, B, r]; lat: [N, B-1, r];
 * u_out: [N, B, r] or NULL (the mixer output, for tests).                                      */
void xo_latent(const float* w1, const float* in_proj, const double* L, const float* w_gate,
               const float* w_up, const float* w_down, int B, int r, int M, int64_t V,
               const int64_t* blk, const int64_t* am1, const double* xh, int N, double* lat,
               double* u_out) {
  xo_latent_weights w = {B, r, M, V, w1, in_proj, L, w_gate, w_up, w_down};
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)B * r);
    double* u = (double*)malloc(sizeof(double) * (size_t)B * r);
    double* a = (double*)malloc(sizeof(double) * (size_t)M);
#pragma omp for schedule(dynamic)
    for (int n = 0; n < N; ++n)
      latent_block(&w, blk + (size_t)n * B, am1[n], xh + (size_t)n * B * r,
                   lat + (size_t)n * (B - 1) * r, u_out ? u_out + (size_t)n * B * r : NULL, x, u,
                   a);
    free(x);
    free(u);
    free(a);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Full-vocabulary readout and argmax (qwen3_xpress, refine_bias and the full-vocab loop of
 * jacobi_refine_greedy; kernels page, module docstring):
 *   logit[p, v] = base[p, v] + sum_i lat[p, i] * w2[v, i],   best[p] = argmax_v logit[p, v]
 * lat: [rows, r]; w2: [V, r]; base: [rows, V] stride ld. gap (nullable): best minus the largest
 * logit at any other id. best_val (nullable): the winning logit.                               */
void xo_readout_argmax(const double* lat, const float* w2, const float* base, int64_t ld,
                       int64_t rows, int64_t V, int r, int64_t* best, double* gap,
                       double* best_val) {
#pragma omp parallel
  {
    double* logit = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic)
    for (int64_t p = 0; p < rows; ++p) {
      const double* lp = lat + p * (int64_t)r;
      for (int64_t v = 0; v < V; ++v) {
        double s = 0.0;
        for (int i = 0; i < r; ++i) s += lp[i] * (double)w2[v * (int64_t)r + i];
        logit[v] = (double)base[p * ld + v] + s;
      }
      best[p] = argmax_with_gap(logit, V, gap ? gap + p : NULL);
      if (best_val) best_val[p] = logit[best[p]];
    }
    free(logit);
  }
}

/* Top-C readout and argmax (qwen3_xpress, top-C loop of jacobi_refine_greedy; kernels page,
 * _xpress_topc_argmax_to_blk_kernel): only the row's candidates are scored,
 *   logit[p, k] = base[p, cand[p, k]] + sum_i lat[p, i] * w2[cand[p, k], i]
 * and the winner is returned as a vocabulary id; ties go to the lowest vocabulary id.
 * cand: [rows, c] (c = min(C, V)).                                                            */
void xo_readout_argmax_topc(const double* lat, const float* w2, const float* base, int64_t ld,
                            const int64_t* cand, int64_t rows, int c, int r, int64_t* best,
                            double* gap, double* best_val) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < rows; ++p) {
    const double* lp = lat + p * (int64_t)r;
    const int64_t* cp = cand + p * (int64_t)c;
    int64_t win = -1;
    double wv = -INFINITY, second = -INFINITY;
    for (int k = 0; k < c; ++k) {
      int64_t id = cp[k];
      double s = 0.0;
      for (int i = 0; i < r; ++i) s += lp[i] * (double)w2[id * (int64_t)r + i];
      double lv = (double)base[p * ld + id] + s;
      if (win < 0 || lv > wv || (lv == wv && id < win)) {
        if (win >= 0) second = (wv > second) ? wv : second;
        win = id;
        wv = lv;
      } else if (lv > second) {
        second = lv;
      }
    }
    best[p] = win;
    if (gap) gap[p] = (c > 1) ? wv - second : INFINITY;
    if (best_val) best_val[p] = wv;
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Jacobi passes (qwen3_xpress, jacobi_refine_greedy): each pass computes every slot's latent from
 * the block as it stood at the start of the pass, scores it, and then writes every slot's winner
 * back, blk[n, b] = best[n*(B-1) + b-1] for b >= 1. With stop_at_fixed_point the loop ends after
 * the first pass that changes no slot (that pass is counted). Returns the passes run.
 * blk: [N, B] in/out. cand: NULL for the full vocabulary, else [rows, c].
 * hist_blk (nullable): [K+1, N, B] blocks before the first pass and after each pass.
 * hist_gap (nullable): [K, rows] the oracle's top-2 gap of every row in every pass.            */
int xo_jacobi(const float* w1, const float* in_proj, const double* L, const float* w_gate,
              const float* w_up, const float* w_down, const float* w2, int B, int r, int M,
              int64_t V, const double* xh, const float* base, int64_t ld, const int64_t* am1,
              int N, const int64_t* cand, int c, int K, int stop_at_fixed_point, int64_t* blk,
              int64_t* hist_blk, double* hist_gap) {
  int64_t rows = (int64_t)N * (B - 1);
  double* lat = (double*)malloc(sizeof(double) * (size_t)rows * r);
  int64_t* best = (int64_t*)malloc(sizeof(int64_t) * (size_t)rows);
  double* gap = (double*)malloc(sizeof(double) * (size_t)rows);
  if (hist_blk) memcpy(hist_blk, blk, sizeof(int64_t) * (size_t)N * B);
  int passes = 0;
  for (int p = 0; p < K; ++p) {
    xo_latent(w1, in_proj, L, w_gate, w_up, w_down, B, r, M, V, blk, am1, xh, N, lat, NULL);
    if (cand)
      xo_readout_argmax_topc(lat, w2, base, ld, cand, rows, c, r, best, gap, NULL);
    else
      xo_readout_argmax(lat, w2, base, ld, rows, V, r, best, gap, NULL);
    int changed = 0;
    for (int n = 0; n < N; ++n)
      for (int b = 1; b < B; ++b) {
        int64_t nb = best[(int64_t)n * (B - 1) + b - 1];
        if (blk[(size_t)n * B + b] != nb) changed = 1;
        blk[(size_t)n * B + b] = nb;
      }
    ++passes;
    if (hist_blk) memcpy(hist_blk + (size_t)(p + 1) * N * B, blk, sizeof(int64_t) * (size_t)N * B);
    if (hist_gap) memcpy(hist_gap + (size_t)p * rows, gap, sizeof(double) * (size_t)rows);
    if (stop_at_fixed_point && !changed) break;
  }
  free(lat);
  free(best);
  free(gap);
  return passes;
}

/* ------------------------------------------------------------------------------------------ */
/* Slot-by-slot sequential greedy decode, by brute force: for b = 1..B-1 the latent of the whole
 * block is recomputed from the tokens decided so far, with every undecided slot filled with
 * `filler` tokens, and slot b takes the argmax of its readout. Independent of the Jacobi loop.
 * Returns in out[N, B] the decoded block (out[n, 0] = anchor[n]). filler: [N, B].              */
void xo_sequential_greedy(const float* w1, const float* in_proj, const double* L,
                          const float* w_gate, const float* w_up, const float* w_down,
                          const float* w2, int B, int r, int M, int64_t V, const double* xh,
                          const float* base, int64_t ld, const int64_t* anchor,
                          const int64_t* am1, int N, const int64_t* cand, int c,
                          const int64_t* filler, int64_t* out) {
  xo_latent_weights w = {B, r, M, V, w1, in_proj, L, w_gate, w_up, w_down};
  double* x = (double*)malloc(sizeof(double) * (size_t)B * r);
  double* u = (double*)malloc(sizeof(double) * (size_t)B * r);
  double* a = (double*)malloc(sizeof(double) * (size_t)M);
  double* lat = (double*)malloc(sizeof(double) * (size_t)(B - 1) * r);
  int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
  for (int n = 0; n < N; ++n) {
    for (int b = 0; b < B; ++b) cur[b] = filler[(size_t)n * B + b];
    cur[0] = anchor[n];
    for (int b = 1; b < B; ++b) {
      latent_block(&w, cur, am1[n], xh + (size_t)n * B * r, lat, NULL, x, u, a);
      int64_t p = (int64_t)n * (B - 1) + b - 1;
      int64_t tok;
      if (cand)
        xo_readout_argmax_topc(lat + (size_t)(b - 1) * r, w2, base + p * ld, 0, cand + p * c,
                               1, c, r, &tok, NULL, NULL);
      else
        xo_readout_argmax(lat + (size_t)(b - 1) * r, w2, base + p * ld, 0, 1, V, r, &tok, NULL,
                          NULL);
      cur[b] = tok;
    }
    for (int b = 0; b < B; ++b) out[(size_t)n * B + b] = cur[b];
  }
  free(x);
  free(u);
  free(a);
  free(lat);
  free(cur);
}
