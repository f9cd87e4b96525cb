// Host-side launchers of the XPress pass kernels. Shapes are validated by the C-ABI layer
// (xpress_api.hip) before any of these is called; each launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xpress {

// Readout partials per row: the vocabulary is cut into contiguous ranges of 32-id steps, at most
// min(256, ceil(V/32)) of them (fewer above 512 rows: about one workgroup per CU either way);
// the readout kernel leaves one (max, lowest id) partial per (row, range).
int readout_tiles(int64_t V, int rows);

// K1a: split-K partials of hdg[m, j] = sum_k h[m, k] * Wcat[j, k], Wcat = [down_h; down_g],
// m < NB = N*B, j < 2r; scratch [hidden_splits, NB, 2r] fp32.
int hidden_splits(int NB, int H, int r);
int hidden_chunks_per_split(int NB, int H, int r);
size_t hidden_scratch_bytes(int NB, int H, int r);
size_t hidden_scratch_bytes_any_h(int NB, int r);
hipError_t launch_hidden_gemm(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                              int NB, int H, int r, float* part, hipStream_t s);
// K1b: reduce the partials (fixed order), then
// xh[n, b] = in_proj[:, :r] . hdg[n, b, :r] + in_proj[:, r:2r] . mean_b hdg[n, b, r:]; `part` is
// the scratch of launch_hidden_gemm (hidden_scratch_bytes long).
// K1a + K2 in one launch (independent): the hidden GEMM's tiles and the starting block's rows.
// With zero_flags (nullable) it also clears the step's nzero pass flags.
hipError_t launch_step_start(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                             int NB, int H, int r, float* part, const uint16_t* base, int64_t ld,
                             const int64_t* anchor, int N, int B, int64_t V, int64_t* blk,
                             hipStream_t s, int32_t* zero_flags = nullptr, int nzero = 0);
hipError_t launch_hidden_project(const float* part, int H, const uint16_t* in_proj, int N, int B,
                                 int r, float* xh, hipStream_t s);
// K2: blk[n, 0] = anchor[n]; blk[n, b] = argmax_v base[n*(B-1)+b-1, v].
hipError_t launch_initial_block(const uint16_t* base, int64_t ld, const int64_t* anchor, int N,
                                int B, int64_t V, int64_t* blk, hipStream_t s);
// K4: latent stage of one pass (three kernels); scratch holds u (fp32 and bf16) and s (bf16).
size_t latent_scratch_bytes(int N, int r, int M);
// Steps 1-5 of the latent. With part != nullptr (inside a step, pass >= 1) the mix kernel first
// reduces the previous pass's range-major partials into blk for its block and raises
// flags[pass-1] on a change; blk is then written. Otherwise blk is only read. lat is row-major
// [N*(B-1), r], or with lat_frag in the readout's fragment order (lat_frag_offset; the buffer
// then holds ceil(N*(B-1)/32) whole 32-row tiles).
hipError_t launch_latent(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                         const float* xh, const uint16_t* w1, const uint16_t* in_proj,
                         const uint16_t* mix_L, const uint16_t* w_gate, const uint16_t* w_up,
                         const uint16_t* w_down, int N, int B, int r, int M, int64_t V,
                         uint16_t* lat, void* scratch, int32_t* flags, int pass, hipStream_t s,
                         bool lat_frag = false);
// K4 from the projected embedding table w1p (launch_fold_embedding), two launches: the
// per-(block, 64-unit slice) shares of the latent, then their sum into lat (skipped with
// with_sum = false, for a consumer that sums the shares itself). dpart: [N, M/64, 16,
// r] fp32 shares (latent_fused_scratch_bytes). part / blk / flags as in launch_latent.
int share_slices(int N, int M);  // latent share workgroups per block (table path)
size_t latent_fused_scratch_bytes(int N, int r, int M);
hipError_t launch_latent_fused(const uint2* part, int ntiles, int64_t* blk, const int64_t* am1,
                               const float* xh, const float* w1p, const uint16_t* mix_L,
                               const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, int N, int B, int r, int M, int64_t V,
                               uint16_t* lat, float* dpart, int32_t* flags, int pass,
                               hipStream_t s, bool with_sum = true, bool lat_frag = false);
// w1p[v, c] = sum_k in_proj[c, 2r + k] * w1[v, k], fp32 [V, r].
hipError_t launch_fold_embedding(const uint16_t* w1, const uint16_t* in_proj, int r, int64_t V,
                                 float* w1p, hipStream_t s);
// K5: per (vocabulary range, row) partial argmax of base + lat . w2^T; part: [ntiles, rows],
// range-major (part[t * rows + p]). lat row-major, or with lat_frag in fragment order.
hipError_t launch_readout_partial(const uint16_t* lat, const uint16_t* w2, const uint16_t* base,
                                  int64_t ld, int rows, int64_t V, int r, uint2* part,
                                  const int32_t* flags, int pass, hipStream_t s,
                                  bool lat_frag = false);
// K6: per-row reduce of the partials into blk[n, 1 + p % (B-1)].
// With passes_run (nullable; the last pass of a step, pass = K-1), also writes the number of
// passes that ran, as launch_count_passes would.
hipError_t launch_argmax_reduce(const uint2* part, int ntiles, int rows, int B, int64_t* blk,
                                int32_t* changed, int32_t* pass_flags, int pass, hipStream_t s,
                                int32_t* passes_run = nullptr);
// K3: top-C candidate selection (+ base_c) and the w2 gather. With blk non-null the selection
// also writes the starting block: each row's best candidate into blk[n, 1 + p % (B-1)] and the
// anchor into blk[n, 0].
// cmax (nullable, 16-byte aligned, topc_select_scratch_bytes long; 0 bytes for rows of up to
// 153,600 ids, which keep them in LDS): per-chunk maxima that let the selection's second pass
// re-read only the chunks that can hold an answer.
hipError_t launch_topc_select(const uint16_t* base, int64_t ld, int rows, int64_t V, int c,
                              int64_t* cand, uint16_t* base_c, const int64_t* anchor, int64_t* blk,
                              int B, uint16_t* cmax, hipStream_t s);
size_t topc_select_scratch_bytes(int rows, int64_t V);
// K1a + K3's selection in one launch (independent): the hidden GEMM's tiles (into part, as
// launch_hidden_gemm) and every draft row's selection (as launch_topc_select, with blk and
// anchor nullable alike).
hipError_t launch_topc_start(const uint16_t* h, const uint16_t* down_h, const uint16_t* down_g,
                             int NB, int H, int r, float* part, const uint16_t* base, int64_t ld,
                             int rows, int64_t V, int c, int64_t* cand, uint16_t* base_c,
                             const int64_t* anchor, int64_t* blk, int B, uint16_t* cmax,
                             hipStream_t s, int32_t* zero_flags = nullptr, int nzero = 0);
hipError_t launch_topc_gather(const int64_t* cand, const uint16_t* w2, int rows, int c, int r,
                              uint16_t* w2c, hipStream_t s);
// K7: top-C GEMV + argmax + candidate -> vocabulary id -> blk. The candidates' rows are
// table[cand[p, k]] with by_id (table = w2 [V, r]), else the gathered table[p, k] (table = w2c
// [rows, c, r]). The latent rows come from lat (bf16), or, with shares != nullptr, from the nsh
// slice shares the latent share kernel leaves ([N, nsh, 16, r] fp32), summed as the latent sum
// kernel would (same bits).
hipError_t launch_topc_readout(const uint16_t* lat, const float* shares, int nsh,
                               const uint16_t* table, bool by_id, const uint16_t* base_c,
                               const int64_t* cand, int rows, int B, int r, int c, int64_t* blk,
                               int32_t* changed, int32_t* pass_flags, int pass, hipStream_t s);
// mix_L = bf16(raw * tril + I), per channel.
hipError_t launch_fold_mixer(const uint16_t* raw, int r, int B, uint16_t* mix_L, hipStream_t s);
// blk[n, 0] = anchor[n] (the step without the argmax start).
hipError_t launch_set_anchor(const int64_t* anchor, int N, int B, int64_t* blk, hipStream_t s);
// Step bookkeeping: zero the per-pass change flags; count the passes that ran.
hipError_t launch_flags_reset(int32_t* flags, int n, hipStream_t s);
hipError_t launch_count_passes(const int32_t* flags, int K, int stop, int32_t* passes_run,
                               hipStream_t s);

}  // namespace xpress
